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
//    others write (m, l, o) partials that decode_merge_kernel, launched next on
//    the same stream, combines (the kernel boundary makes the partials visible;
//    no cross-workgroup atomics: same-address device-scope atomics serialise
//    across the chip's XCDs).
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

  // wave w takes pages p_begin + w, + 4, ...; up to kBatch of them are loaded
  // before any is used so that many 4 KiB page reads are in flight per wave
  constexpr int kBatch = 4;
  for (int p0 = p_begin + wave; p0 < p_end; p0 += 4 * kBatch) {
    bf16x8 kf[kBatch][NQ];
    u32x2 vf[kBatch][NDB];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      // pages past the split's end reload its last page (no extra HBM traffic,
      // no branch between the loads) and are skipped below
      const int p = min(p0 + 4 * j, p_end - 1);
      const int64_t phys = trow[p];
      const uint16_t* kpage = kpool + (phys * Hkv + g) * (kPage * D);
      const uint16_t* vpage = vpool + (phys * Hkv + g) * (D * kPage);
#pragma unroll
      for (int c = 0; c < NQ; ++c)
        kf[j][c] = *reinterpret_cast<const bf16x8*>(kpage + c16 * D + c * 32 + grp * 8);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        vf[j][db] = *reinterpret_cast<const u32x2*>(vpage + (db * 16 + c16) * kPage + grp * 4);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int p = p0 + 4 * j;
      if (p >= p_end) break;
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NQ; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[j][c], qf[c], s, 0, 0, 0);
      const int key0 = p * kPage + grp * 4;   // keys of this lane's rows: key0 + i
      if (p * kPage + kPage > T) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key0 + i >= T) s[i] = -INFINITY;
        // stale slots past the length: zero their values so 0 * NaN never occurs
        const uint32_t k01 = (key0 < T ? 0x0000ffffu : 0u) | (key0 + 1 < T ? 0xffff0000u : 0u);
        const uint32_t k23 = (key0 + 2 < T ? 0x0000ffffu : 0u) | (key0 + 3 < T ? 0xffff0000u : 0u);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          vf[j][db][0] &= k01;
          vf[j][db][1] &= k23;
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
        o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vf[j][db]), pb, o[db], 0, 0,
                                                          0);
      }
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
  const bool hv2 = hl2 < G;
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
  uint16_t* orow = static_cast<uint16_t*>(a.o) + b * a.o_s0 + static_cast<int64_t>(h2) * a.o_s1;
  if (nsplit == 1) {
    if (!hv2) return;
    const float inv = 1.f / L;
    for (int dd = dl; dd < D; dd += 16) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) acc += red_o[w][hh][dd] * sc[w];
      orow[dd] = f32_to_bf16(acc * inv);
    }
    return;
  }

  // several splits: write this split's (m, l, o); decode_merge_kernel, the
  // next launch on the stream, combines them.  Partials of one (sequence,
  // blockIdx.y) are contiguous: [split][head in chunk][D + 4] floats, o in
  // 0..D-1 and (m, l) at D, D+1.
  if (!hv2) return;
  constexpr int kRec = D + 4;
  const int Gc = min(16, G - hcb * 16);
  float* rec = a.part_o + ((static_cast<int64_t>(a.split_off[b]) * gridDim.y +
                            static_cast<int64_t>(blockIdx.y) * nsplit) * 16 +
                           static_cast<int64_t>(split) * Gc + hh) * kRec;
  for (int dd = dl; dd < D; dd += 16) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) acc += red_o[w][hh][dd] * sc[w];
    rec[dd] = acc;
  }
  if (dl == 0) {
    rec[D] = M;
    rec[D + 1] = L;
  }
}

// grid: x = sequence, y = query head; one thread per output dimension.
// Combines the split partials of sequences that needed more than one split:
// with M = max_s m_s, o = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
template <int D>
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeArgs a) {
  constexpr int kRec = D + 4;
  constexpr int kMaxSplit = 128;
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const int nsplit = a.split_off[b + 1] - a.split_off[b];
  if (nsplit <= 1) return;
  const int G = a.Hq / a.Hkv;
  const int hchunks = (G + 15) >> 4;
  const int gy = a.Hkv * hchunks;
  const int g = h / G;
  const int hl = h - g * G;
  const int hcb = hl >> 4;
  const int hh = hl & 15;
  const int Gc = min(16, G - hcb * 16);
  const int y = g * hchunks + hcb;
  const float* region = a.part_o + (static_cast<int64_t>(a.split_off[b]) * gy + static_cast<int64_t>(y) * nsplit) *
                                       (16 * kRec);
  __shared__ float s_w[kMaxSplit];
  __shared__ float s_red[2][4];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = t >> 6;
  float m = -INFINITY, l = 0.f;
  if (t < nsplit) {
    const float* r = region + (static_cast<int64_t>(t) * Gc + hh) * kRec;
    m = r[D];
    l = r[D + 1];
  }
  float M = m;
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) s_red[0][wv] = M;
  __syncthreads();
  M = fmaxf(s_red[0][0], s_red[0][1]);
  const float w = t < nsplit ? __builtin_amdgcn_exp2f(m - M) : 0.f;
  if (t < nsplit) s_w[t] = w;
  float L = l * w;
  for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
  if (lane == 0) s_red[1][wv] = L;
  __syncthreads();
  L = s_red[1][0] + s_red[1][1];
  if (t >= D) return;
  const float* col = region + static_cast<int64_t>(hh) * kRec + t;
  const int64_t stride = static_cast<int64_t>(Gc) * kRec;
  float acc = 0.f;
  int sp = 0;
  for (; sp + 16 <= nsplit; sp += 16) {
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = col[(sp + k) * stride];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc += v[k] * s_w[sp + k];
  }
  for (; sp < nsplit; ++sp) acc += col[sp * stride] * s_w[sp];
  uint16_t* out = static_cast<uint16_t*>(a.o) + b * a.o_s0 + static_cast<int64_t>(h) * a.o_s1;
  out[t] = f32_to_bf16(acc / L);
}

hipError_t launch_decode_bf16(const DecodeArgs& a, int total_splits, bool merge, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int hchunks = (G + 15) / 16;
  dim3 grid(total_splits, a.Hkv * hchunks);
  if (a.d == 128)
    hipLaunchKernelGGL(decode_bf16_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(decode_bf16_kernel<64>, grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !merge) return e;
  if (a.d == 128)
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(a.nseq, a.Hq), dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(a.nseq, a.Hq), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace gqa
