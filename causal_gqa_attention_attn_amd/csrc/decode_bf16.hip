// bfloat16 split-T decode attention over the paged cache.
//
// What it computes (page "模型执行：从 token 到 Prefill 与 Decode", prefill and
// decode shapes; page "KV Cache 与 Prefill/Decode 推理路径", single-token
// decode needs no mask): one new query per sequence, at position T-1, attends
// to all T cached slots of its KV head g(h) = floor(h*Hkv/Hq):
//   o[b,h] = sum_{j<T} softmax_j(<rot(q), k_used[g,j]>/sqrt(d)) v[g,j].
//
// How (memory-bound; every K/V byte is read from HBM once per step):
//  * one workgroup = (sequence, split of consecutive pages, kv head, up to 16
//    query heads of its group); its four waves take the split's pages in turn;
//  * per page: S^T[16 keys x 16 heads] = K q^T on v_mfma_f32_16x16x32_bf16 with
//    the K rows loaded straight from the page (16-byte loads, the whole page is
//    one contiguous 4 KiB run for d=128), then O^T[d x heads] += V^T P^T on
//    v_mfma_f32_16x16x16_bf16 with V^T read straight from the d-major page;
//    the score accumulator is already the B operand of the second product;
//  * online softmax in base 2 per head; the four waves and then the splits
//    are combined with the log-sum-exp rule: with M = max_s m_s,
//    O = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M);
//  * a sequence whose pages fit one split writes its output directly; the
//    others write (m, l, o) partials that decode_merge_kernel combines.
#include "common.hpp"
#include "device.hpp"

namespace gqa {

template <int D>
__global__ __launch_bounds__(256) void decode_bf16_kernel(DecodeArgs a) {
  constexpr int NQ = D / 32;      // k-steps of the score product
  constexpr int NDB = D / 16;     // 16-row blocks of the output
  __shared__ float red_m[4][16];
  __shared__ float red_l[4][16];
  __shared__ float red_o[4][16][D + 4];

  const int G = a.Hq / a.Hkv;
  const int hchunks = (G + 15) >> 4;
  const int g = blockIdx.y / hchunks;
  const int hcb = blockIdx.y - g * hchunks;
  int b = 0;
  while (b + 1 < a.nseq && a.split_off[b + 1] <= static_cast<int>(blockIdx.x)) ++b;
  const int split = blockIdx.x - a.split_off[b];
  const int nsplit = a.split_off[b + 1] - a.split_off[b];
  const int seq = a.meta.seq[b];
  const int T = a.meta.total[b];
  const int qpos = a.meta.start[b];
  const int npages = (T + kPage - 1) / kPage;
  const int p_begin = split * a.pages_per_split;
  const int p_end = min(npages, p_begin + a.pages_per_split);

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;
  const int c16 = lane & 15;
  const int hl = hcb * 16 + c16;           // head within the group held by this lane column
  const bool hvalid = hl < G;
  const int h = g * G + hl;

  // rotated query as B operand: lane (head c16, grp) holds dims 32c + 8*grp + 0..7
  bf16x8 qf[NQ];
  {
    float x[NQ][8];
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + b * a.q_s0 + static_cast<int64_t>(h) * a.q_s1;
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (hvalid) w = *reinterpret_cast<const u32x4*>(qrow + c * 32 + grp * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[c][2 * e] = __uint_as_float(w[e] << 16);
        x[c][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    }
    if (a.rope && hvalid) {
      const float* rrow = a.rope + static_cast<int64_t>(qpos) * D;
#pragma unroll
      for (int c = 0; c < NQ / 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = c * 32 + grp * 8 + e;
          float lo, hi;
          rotate_pair(x[c][e], x[c + NQ / 2][e], rrow[2 * i], rrow[2 * i + 1], lo, hi);
          x[c][e] = lo;
          x[c + NQ / 2][e] = hi;
        }
    }
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[c][2 * e], x[c][2 * e + 1]);
      qf[c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const uint16_t* kpool = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* vpool = static_cast<const uint16_t*>(a.v_pool);
  const int32_t* trow = a.table + static_cast<int64_t>(seq) * a.table_w;
  const int Hkv = a.Hkv;
  const float sl2 = a.scale_log2;

  f32x4 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -1e30f;
  float l_run = 0.f;

  for (int p = p_begin + wave; p < p_end; p += 4) {
    const int64_t phys = trow[p];
    const uint16_t* kpage = kpool + (phys * Hkv + g) * (kPage * D);
    const uint16_t* vpage = vpool + (phys * Hkv + g) * (D * kPage);
    bf16x8 kf[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c)
      kf[c] = *reinterpret_cast<const bf16x8*>(kpage + c16 * D + c * 32 + grp * 8);
    u32x2 vf[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      vf[db] = *reinterpret_cast<const u32x2*>(vpage + (db * 16 + c16) * kPage + grp * 4);

    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NQ; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], qf[c], s, 0, 0, 0);
    const int key0 = p * kPage + grp * 4;   // keys of this lane's rows: key0 + i
    const bool tail = p * kPage + kPage > T;
    if (tail) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (key0 + i >= T) s[i] = -INFINITY;
      // stale slots past the length: zero their values so 0 * NaN never occurs
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint32_t k01 = (key0 < T ? 0x0000ffffu : 0u) | (key0 + 1 < T ? 0xffff0000u : 0u);
        const uint32_t k23 = (key0 + 2 < T ? 0x0000ffffu : 0u) | (key0 + 3 < T ? 0xffff0000u : 0u);
        vf[db][0] &= k01;
        vf[db][1] &= k23;
      }
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(s[i], sl2, -m_new));
    l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    s16x4 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[i] = __builtin_bit_cast(short, static_cast<__bf16>(pr[i]));
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      o[db] *= alpha;
      o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vf[db]), pb, o[db], 0, 0, 0);
    }
  }

  // combine the four waves: lane (head c16, grp) holds o rows d = 16*db + 4*grp + i
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (grp == 0) {
    red_m[wave][c16] = m_run;
    red_l[wave][c16] = l_tot;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) red_o[wave][c16][db * 16 + grp * 4 + i] = o[db][i];
  __syncthreads();

  // 256 threads: head column hh = tid / 16, 16 threads per head over d
  const int hh = threadIdx.x >> 4;
  const int dl = threadIdx.x & 15;
  const int hl2 = hcb * 16 + hh;
  if (hl2 >= G) return;
  const int h2 = g * G + hl2;
  float M = red_m[0][hh];
#pragma unroll
  for (int w = 1; w < 4; ++w) M = fmaxf(M, red_m[w][hh]);
  float sc[4];
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    sc[w] = __builtin_amdgcn_exp2f(red_m[w][hh] - M);
    L += red_l[w][hh] * sc[w];
  }
  if (nsplit == 1) {
    const float inv = 1.f / L;
    uint16_t* orow = static_cast<uint16_t*>(a.o) + b * a.o_s0 + static_cast<int64_t>(h2) * a.o_s1;
    for (int dd = dl; dd < D; dd += 16) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += red_o[w][hh][dd] * sc[w];
      orow[dd] = f32_to_bf16(acc * inv);
    }
  } else {
    const int64_t slot = static_cast<int64_t>(a.split_off[b] + split) * a.Hq + h2;
    float* po = a.part_o + slot * D;
    for (int dd = dl; dd < D; dd += 16) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += red_o[w][hh][dd] * sc[w];
      po[dd] = acc;
    }
    if (dl == 0) {
      a.part_ml[slot * 2] = M;
      a.part_ml[slot * 2 + 1] = L;
    }
  }
}

// grid: x = sequence, y = query head.  Combines the split partials of
// sequences that needed more than one split.
__global__ __launch_bounds__(128) void decode_merge_kernel(MergeArgs a) {
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const int n = a.split_off[b + 1] - a.split_off[b];
  if (n <= 1) return;
  const int64_t base = a.split_off[b];
  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, a.part_ml[((base + s) * a.Hq + h) * 2]);
  float L = 0.f;
  for (int s = 0; s < n; ++s) {
    const int64_t slot = (base + s) * a.Hq + h;
    L += a.part_ml[slot * 2 + 1] * __builtin_amdgcn_exp2f(a.part_ml[slot * 2] - M);
  }
  const float inv = 1.f / L;
  uint16_t* orow = static_cast<uint16_t*>(a.o) + b * a.o_s0 + static_cast<int64_t>(h) * a.o_s1;
  for (int dd = threadIdx.x; dd < a.d; dd += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < n; ++s) {
      const int64_t slot = (base + s) * a.Hq + h;
      acc += a.part_o[slot * a.d + dd] * __builtin_amdgcn_exp2f(a.part_ml[slot * 2] - M);
    }
    orow[dd] = f32_to_bf16(acc * inv);
  }
}

hipError_t launch_decode_bf16(const DecodeArgs& a, int total_splits, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int hchunks = (G + 15) / 16;
  dim3 grid(total_splits, a.Hkv * hchunks);
  if (a.d == 128)
    hipLaunchKernelGGL(decode_bf16_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(decode_bf16_kernel<64>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const MergeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(decode_merge_kernel, dim3(a.nseq, a.Hq), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace gqa
