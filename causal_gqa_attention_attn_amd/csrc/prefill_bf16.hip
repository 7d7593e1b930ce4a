// bfloat16 causal grouped-query prefill attention on the gfx950 matrix cores.
//
// What it computes (page "Prefill：整层状态演化与 KV 建立", sections 2.2-2.3):
// for every valid query token at position p of sequence b and query head h,
//   O[b,h,p] = sum_{j<=p} softmax_j(<rot(q), k_used[g(h), j]> / sqrt(d)) v[g(h), j]
// with g(h) = floor(h*Hkv/Hq), over the cache slots written for the sequence
// (slot = position; with an older prefix in the cache this is the incremental
// prefill of page "KV Cache 与 Prefill/Decode 推理路径": the prefix is wholly
// visible, the new block lower-triangular).  Padding rows of O are zeroed.
//
// How (gfx950 design, not a translation of any page's kernel):
//  * one workgroup = (kv head g, up to 8 query heads of its group, sequence,
//    32 query tokens); one wave per query head, so every K/V tile staged in LDS
//    is shared by all query heads of the group (the head map is an index, the
//    cache is never replicated);
//  * S^T = K q^T on v_mfma_f32_32x32x16_bf16 with keys as rows: each lane owns
//    one query column, so row max and row sum stay inside a lane plus one
//    exchange with the lane 32 away;
//  * K rows are fed to the matrix core in a fixed permutation so that the score
//    accumulator already has the register layout of the B operand of
//    O^T += V^T P^T (no shuffle of P);
//  * V pages are stored d-major, so V^T tiles are staged with plain 16-byte
//    copies;
//  * online softmax in base 2 with the 1/sqrt(d)*log2(e) scale folded into one
//    multiply-add; the running maximum starts at a finite sentinel so a tile in
//    which every key is masked never evaluates (-inf) - (-inf);
//  * key tiles wholly in the future of the block are never loaded (the loop
//    ends at the block's last query position); only tiles crossing the
//    diagonal are masked, by select;
//  * slots at or beyond the written length are zero-filled in LDS, so stale or
//    poisoned cache memory never meets a zero weight (0 * NaN);
//  * blocks are dispatched heaviest (last) query tile first.
#include "common.hpp"
#include "device.hpp"

namespace gqa {

namespace {

// Key (or head-dim) row fed to MFMA row r: keeps the accumulator of rows
// 8*(i/4) + 4*half + i%4 equal to keys 16*(i/8) + 8*half + i%8.
__device__ __forceinline__ int perm32(int r) {
  return ((r >> 4) << 4) + (((r >> 2) & 1) << 3) + (((r >> 3) & 1) << 2) + (r & 3);
}

}  // namespace

template <int D>
__global__ __launch_bounds__(512) void prefill_bf16_kernel(AttnArgs a) {
  constexpr int KT = 64;          // keys per staged tile
  constexpr int KPAD = D + 8;     // LDS row stride of K (elements)
  constexpr int VPAD = KT + 8;    // LDS row stride of V^T
  constexpr int NC = D / 16;      // k-steps of the score product
  constexpr int NDB = D / 32;     // 32-row blocks of the output
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[KT * KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[D * VPAD];

  const int G = a.Hq / a.Hkv;
  const int chunks = (G + 7) >> 3;
  const int g = blockIdx.x / chunks;
  const int hc = blockIdx.x - g * chunks;
  const int b = blockIdx.y;
  const int tile = gridDim.z - 1 - blockIdx.z;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int heads_here = min(8, G - hc * 8);
  const bool active = wave < heads_here;
  const int h = g * G + hc * 8 + wave;

  const int seq = a.meta.seq[b];
  const int c0 = a.meta.start[b];
  const int nb = a.meta.count[b];
  const int r0 = a.meta.row0[b];
  const int total = a.meta.total[b];

  uint16_t* obase = static_cast<uint16_t*>(a.O) + b * a.o_s0 + static_cast<int64_t>(h) * a.o_s1;

  // padding rows of this block's rectangular range -> 0
  if (active) {
    const int rlo = tile * 32;
    const int rhi = min(a.n_rect, rlo + 32);
    for (int idx = lane; idx < 32 * (D / 8); idx += 64) {
      const int rr = rlo + idx / (D / 8);
      const int ch = idx % (D / 8);
      if (rr < rhi && (rr < r0 || rr >= r0 + nb)) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(obase + static_cast<int64_t>(rr) * a.o_s2 + ch * 8) = z;
      }
    }
  }

  const int t0 = tile * 32;
  if (t0 >= nb) return;
  const int qn = min(32, nb - t0);
  const bool qvalid = col < qn;
  const int pos = c0 + t0 + col;

  // rotated queries as B operands: lane holds dims 16c + 8*half + 0..7 of its query
  bf16x8 qf[NC];
  if (active) {
    float x[NC][8];
    const uint16_t* qrow = static_cast<const uint16_t*>(a.Q) + b * a.q_s0 + static_cast<int64_t>(h) * a.q_s1 +
                           static_cast<int64_t>(r0 + t0 + col) * a.q_s2;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qvalid) w = *reinterpret_cast<const u32x4*>(qrow + c * 16 + half * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[c][2 * e] = __uint_as_float(w[e] << 16);
        x[c][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    }
    if (a.rope && qvalid) {
      const float* rrow = a.rope + static_cast<int64_t>(pos) * D;   // (D/2) pairs
#pragma unroll
      for (int c = 0; c < NC / 2; ++c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = c * 16 + half * 8 + e;
          float lo, hi;
          rotate_pair(x[c][e], x[c + NC / 2][e], rrow[2 * i], rrow[2 * i + 1], lo, hi);
          x[c][e] = lo;
          x[c + NC / 2][e] = hi;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[c][2 * e], x[c][2 * e + 1]);
      qf[c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int kv_end = c0 + t0 + qn;            // keys [0, kv_end) can be visible
  const int ntk = (kv_end + KT - 1) / KT;
  const int diag = c0 + t0;                   // smallest query position of the block
  const uint16_t* kpool = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* vpool = static_cast<const uint16_t*>(a.v_pool);
  const int32_t* trow = a.table + static_cast<int64_t>(seq) * a.table_w;
  const int Hkv = a.Hkv;
  const float sl2 = a.scale_log2;

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m_run = -1e30f;     // finite sentinel (log2 units)
  float l_run = 0.f;
  const int krow_l = perm32(col);

  for (int kt = 0; kt < ntk; ++kt) {
    const int kbase = kt * KT;
    __syncthreads();
    for (int ci = threadIdx.x; ci < KT * D / 8; ci += blockDim.x) {
      const int kl = ci / (D / 8);
      const int ch = ci - kl * (D / 8);
      const int key = kbase + kl;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (key < total) {
        const int64_t phys = trow[key >> 4];
        val = *reinterpret_cast<const u32x4*>(kpool + ((phys * Hkv + g) * kPage + (key & 15)) * D + ch * 8);
      }
      *reinterpret_cast<u32x4*>(k_lds + kl * KPAD + ch * 8) = val;
    }
    for (int ci = threadIdx.x; ci < KT * D / 8; ci += blockDim.x) {
      const int pl = ci / (D * 2);
      const int rem = ci - pl * (D * 2);
      const int dd = rem >> 1;
      const int h8 = rem & 1;
      const int key0 = kbase + pl * 16 + h8 * 8;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (key0 < total) {
        const int64_t phys = trow[key0 >> 4];
        val = *reinterpret_cast<const u32x4*>(vpool + ((phys * Hkv + g) * D + dd) * kPage + h8 * 8);
        const int nv = total - key0;
        if (nv < 8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t keep_lo = (2 * e < nv) ? 0x0000ffffu : 0u;
            const uint32_t keep_hi = (2 * e + 1 < nv) ? 0xffff0000u : 0u;
            val[e] &= (keep_lo | keep_hi);
          }
        }
      }
      *reinterpret_cast<u32x4*>(v_lds + dd * VPAD + pl * 16 + h8 * 8) = val;
    }
    __syncthreads();
    if (!active) continue;

    // S^T for 64 keys: two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
      const uint16_t* kr = k_lds + (kb * 32 + krow_l) * KPAD + half * 8;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kr + c * 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[kb], 0, 0, 0);
      }
    }
    if (kbase + KT - 1 > diag) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase + kb * 32 + 16 * (i >> 3) + 8 * half + (i & 7);
          if (key > pos) s[kb][i] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    bf16x8 pf[2][2];
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][i], sl2, -m_new));
        lsum += p;
        pf[kb][i >> 3][i & 7] = static_cast<__bf16>(p);
      }
    l_run += lsum;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
              v_lds + (db * 32 + krow_l) * VPAD + kb * 32 + sub * 16 + half * 8);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][sub], o[db], 0, 0, 0);
        }
  }

  if (!active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  if (qvalid) {
    uint16_t* orow = obase + static_cast<int64_t>(r0 + t0 + col) * a.o_s2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = pack_bf16x2(o[db][sub * 8 + 2 * e] * inv, o[db][sub * 8 + 2 * e + 1] * inv);
        *reinterpret_cast<u32x4*>(orow + db * 32 + sub * 16 + half * 8) = w;
      }
  }
}

hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int chunks = (G + 7) / 8;
  const int waves = G < 8 ? G : 8;
  dim3 grid(a.Hkv * chunks, a.nseq, (a.n_rect + 31) / 32);
  dim3 block(64 * waves);
  if (a.d == 128)
    hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace gqa
