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
// How (a gfx950 design, not a translation of any page's kernel):
//  * one workgroup = 4 waves, one per SIMD, for (kv head g, a chunk of Gc of
//    its query heads, sequence, Tq query tokens).  Its Gc*Tq query rows form
//    row-blocks of 32 (one head, 32 tokens); each wave owns R of them, so every
//    K/V fragment it reads from LDS feeds R matrix-core products, and every K/V
//    tile staged in LDS serves all Gc query heads of the group (the head map is
//    an index; the cache is never replicated);
//  * S^T = K q^T on v_mfma_f32_32x32x16_bf16 with keys as rows: each lane owns
//    one query column, so row maxima and sums stay in a lane plus one exchange
//    with the lane 32 away;
//  * K rows are fed to the matrix core in a fixed permutation so the score
//    accumulator already has the register layout of the B operand of
//    O^T += V^T P^T (no shuffle of P); V pages are stored d-major, so V^T tiles
//    are staged with plain 16-byte copies;
//  * 64-key K/V tiles are double-buffered in LDS: the next tile's global loads
//    are in flight while the current one is used, one barrier per tile;
//  * softmax in base 2 with the 1/sqrt(d)*log2(e) scale folded into one
//    multiply-add, against a fixed reference per query row: the maximum of the
//    row's first 32-key sub-tile (which always holds key 0, visible to every
//    query, so the reference is finite and a fully masked later tile never
//    meets (-inf) - (-inf)).  Unnormalised probabilities 2^(s - ref) and their
//    sums stay exact in float32/bf16 range while no score exceeds the
//    reference by more than 2^64, so the output accumulators are never
//    rescaled in the loop.  Each lane records its largest score; if any lane
//    of the workgroup passes that bound, the workgroup runs the tile loop once
//    more with the recorded maxima as references, which cannot overflow;
//  * key tiles wholly in the future of a workgroup are never loaded; 32-key
//    sub-tiles wholly in the future of a row-block are skipped; masking by
//    select happens only on tiles that cross the diagonal;
//  * slots at or beyond the written length are zero-filled in LDS, so stale or
//    poisoned cache memory never meets a zero weight (0 * NaN);
//  * workgroups are dispatched heaviest (last) query tile first.
#include <type_traits>

#include "common.hpp"
#include "device.hpp"

namespace gqa {

namespace {

// Key (or head-dim) row fed to MFMA row r: keeps the accumulator of rows
// 8*(i/4) + 4*half + i%4 equal to keys 16*(i/8) + 8*half + i%8.
__device__ __forceinline__ int perm32(int r) {
  return ((r >> 4) << 4) + (((r >> 2) & 1) << 3) + (((r >> 3) & 1) << 2) + (r & 3);
}

constexpr int KT = 64;                 // keys per staged tile

template <int D>
struct Smem {
  static constexpr int KPAD = D + 8;   // LDS row stride of K (elements)
  static constexpr int VPAD = KT + 8;  // LDS row stride of V^T
  static constexpr int K_ELEMS = KT * KPAD;
  static constexpr int V_ELEMS = D * VPAD;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
};

}  // namespace

// Template R: row-blocks per wave.  Runtime Gc (heads per workgroup) and TB
// (32-token blocks per workgroup) satisfy Gc * TB == 4 * R.
template <int D, int R>
__global__ __launch_bounds__(256, R == 1 ? 2 : 1) void prefill_bf16_kernel(AttnArgs a, int Gc, int TB) {
  using S = Smem<D>;
  constexpr int NC = D / 16;           // k-steps of the score product
  constexpr int NDB = D / 32;          // 32-row blocks of the output
  constexpr int KCH = KT * D / 8;      // 16-byte chunks of a K (or V) tile
  constexpr int PER_T = KCH / 256;     // chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * S::BUF];

  // kv head fastest: with 8 kv heads, block i lands on XCD i % 8 = its kv head,
  // so each XCD's L2 holds the keys and values of one head
  const int G = a.Hq / a.Hkv;
  const int hc = blockIdx.x / a.Hkv;
  const int g = blockIdx.x - hc * a.Hkv;
  const int b = blockIdx.y;
  const int tile = gridDim.z - 1 - blockIdx.z;
  const int Tq = 32 * TB;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int col = lane & 31;

  const int seq = a.meta.seq[b];
  const int c0 = a.meta.start[b];
  const int nb = a.meta.count[b];
  const int r0 = a.meta.row0[b];
  const int total = a.meta.total[b];
  const int h0 = g * G + hc * Gc;      // first query head of this workgroup

  // padding rows of this workgroup's rectangular range -> 0
  {
    const int rlo = tile * Tq;
    const int rhi = min(a.n_rect, rlo + Tq);
    const int per_row = D / 8;
    for (int idx = threadIdx.x; idx < Gc * Tq * per_row; idx += 256) {
      const int hh = idx / (Tq * per_row);
      const int rem = idx - hh * Tq * per_row;
      const int rr = rlo + rem / per_row;
      const int ch = rem % per_row;
      if (rr < rhi && (rr < r0 || rr >= r0 + nb)) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        uint16_t* op = static_cast<uint16_t*>(a.O) + b * a.o_s0 + static_cast<int64_t>(h0 + hh) * a.o_s1 +
                       static_cast<int64_t>(rr) * a.o_s2 + ch * 8;
        *reinterpret_cast<u32x4*>(op) = z;
      }
    }
  }

  const int t0 = tile * Tq;
  if (t0 >= nb) return;
  const int qn = min(Tq, nb - t0);

  // this wave's row-blocks: head, first token, validity
  int rb_h[R], rb_t[R];
  bool rb_ok[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int rb = wave * R + j;
    rb_h[j] = h0 + rb / TB;
    rb_t[j] = (rb % TB) * 32;          // token offset inside the tile
    rb_ok[j] = rb_t[j] < qn;
  }

  // rotated queries as B operands: lane holds dims 16c + 8*half + 0..7 of its query
  bf16x8 qf[R][NC];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int t = t0 + rb_t[j] + col;
    const bool qv = rb_ok[j] && (rb_t[j] + col < qn);
    float x[NC][8];
    const uint16_t* qrow = static_cast<const uint16_t*>(a.Q) + b * a.q_s0 + static_cast<int64_t>(rb_h[j]) * a.q_s1 +
                           static_cast<int64_t>(r0 + t) * a.q_s2;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qv) w = *reinterpret_cast<const u32x4*>(qrow + c * 16 + half * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[c][2 * e] = __uint_as_float(w[e] << 16);
        x[c][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    }
    if (a.rope && qv) {
      const float* rrow = a.rope + static_cast<int64_t>(c0 + t) * D;    // (D/2) (cos, sin) pairs
#pragma unroll
      for (int c = 0; c < NC / 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = c * 16 + half * 8 + e;
          float lo, hi;
          rotate_pair(x[c][e], x[c + NC / 2][e], rrow[2 * i], rrow[2 * i + 1], lo, hi);
          x[c][e] = lo;
          x[c + NC / 2][e] = hi;
        }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[c][2 * e], x[c][2 * e + 1]);
      qf[j][c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int kv_end = c0 + t0 + qn;            // keys [0, kv_end) can be visible
  const int ntk = (kv_end + KT - 1) / KT;
  const uint16_t* kpool = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* vpool = static_cast<const uint16_t*>(a.v_pool);
  const int32_t* trow = a.table + static_cast<int64_t>(seq) * a.table_w;
  const int Hkv = a.Hkv;
  const float sl2 = a.scale_log2;

  // ---- global -> registers -> LDS staging of one K/V tile.  The tile's
  // four pages are looked up once; a thread's 16-byte chunks fall in known
  // pages, so all its loads issue back to back.  Slots at or past the written
  // length read a valid page and are zeroed afterwards (no branches).
  const int last_page = (total - 1) >> 4;
  u32x4 stg[2 * PER_T];
  auto load_tile = [&](int kt) {
    const int kbase = kt * KT;
    int64_t phys[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) phys[p] = trow[min(kt * 4 + p, last_page)];
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int ci = threadIdx.x + 256 * i;
      const int kl = ci / (D / 8);
      const int ch = ci - kl * (D / 8);
      const int pl = kl >> 4;
      const int64_t ph = pl == 0 ? phys[0] : pl == 1 ? phys[1] : pl == 2 ? phys[2] : phys[3];
      stg[i] = *reinterpret_cast<const u32x4*>(kpool + ((ph * Hkv + g) * kPage + (kl & 15)) * D + ch * 8);
    }
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int ci = threadIdx.x + 256 * i;
      const int pl = ci / (D * 2);
      const int rem = ci - pl * (D * 2);
      const int dd = rem >> 1;
      const int h8 = rem & 1;
      const int64_t ph = pl == 0 ? phys[0] : pl == 1 ? phys[1] : pl == 2 ? phys[2] : phys[3];
      stg[PER_T + i] = *reinterpret_cast<const u32x4*>(vpool + ((ph * Hkv + g) * D + dd) * kPage + h8 * 8);
    }
    if (kbase + KT > total) {            // the tile holds the end of the sequence
#pragma unroll
      for (int i = 0; i < PER_T; ++i) {
        const int ci = threadIdx.x + 256 * i;
        const int key = kbase + ci / (D / 8);
        if (key >= total) stg[i] = u32x4{0u, 0u, 0u, 0u};
        const int pl = ci / (D * 2);
        const int h8 = (ci - pl * (D * 2)) & 1;
        const int key0 = kbase + pl * 16 + h8 * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t keep_lo = (key0 + 2 * e < total) ? 0x0000ffffu : 0u;
          const uint32_t keep_hi = (key0 + 2 * e + 1 < total) ? 0xffff0000u : 0u;
          stg[PER_T + i][e] &= (keep_lo | keep_hi);
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* kl_s = smem + buf * S::BUF;
    uint16_t* vl_s = kl_s + S::K_ELEMS;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int ci = threadIdx.x + 256 * i;
      const int kl = ci / (D / 8);
      const int ch = ci - kl * (D / 8);
      *reinterpret_cast<u32x4*>(kl_s + kl * S::KPAD + ch * 8) = stg[i];
    }
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int ci = threadIdx.x + 256 * i;
      const int pl = ci / (D * 2);
      const int rem = ci - pl * (D * 2);
      const int dd = rem >> 1;
      const int h8 = rem & 1;
      *reinterpret_cast<u32x4*>(vl_s + dd * S::VPAD + pl * 16 + h8 * 8) = stg[PER_T + i];
    }
  };

  f32x16 o[R][NDB];
  float m_ref[R], m_seen[R], l_run[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    m_ref[j] = -INFINITY;              // set from the first sub-tile of the row-block
    m_seen[j] = -INFINITY;
  }
  const int krow_l = perm32(col);
  bool all_ok = true;
#pragma unroll
  for (int j = 0; j < R; ++j) all_ok = all_ok && rb_ok[j];
  bool ovf = false;
  int pass = 0;
  __shared__ int redo;
  // softmax of one 32-key sub-tile for row-block j: mask, row maximum,
  // probabilities against the row's reference, row sum, bf16 B operands
  auto softmax32 = [&](f32x16& sc, int j, int k0, bool msk, bf16x8* pf) {
    if (msk) {
      const int pos = c0 + t0 + rb_t[j] + col;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 16 * (i >> 3) + 8 * half + (i & 7);
        if (key > pos) sc[i] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, sc[i]), sc[i + 1]);
    mx = fmaxf(mx, sc[15]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
    if (pass == 0 && k0 == 0) m_ref[j] = mx;      // first sub-tile of every row-block
    m_seen[j] = fmaxf(m_seen[j], mx);
    ovf |= mx > m_ref[j] + 64.f;
    const float mneg = -m_ref[j];
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sc[i], sl2, mneg));
      lsum += p;
      pf[i >> 3][i & 7] = static_cast<__bf16>(p);
    }
    l_run[j] += lsum;
  };

  auto compute_tile = [&](const uint16_t* kl_s, const uint16_t* vl_s, int kt, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    if constexpr (R == 1) {
      // both 32-key sub-tiles at once: two independent accumulator chains
      const int qlo = c0 + t0 + rb_t[0];
      bool act[2], msk[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int k0 = kt * KT + sub * 32;
        act[sub] = MASKED ? (rb_ok[0] && k0 <= qlo + 31) : true;
        msk[sub] = MASKED && k0 + 31 > qlo;
      }
      f32x16 sc[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[sub][i] = 0.f;
      const uint16_t* kr = kl_s + krow_l * S::KPAD + half * 8;
      if (!MASKED || act[1]) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 k0f = *reinterpret_cast<const bf16x8*>(kr + c * 16);
          const bf16x8 k1f = *reinterpret_cast<const bf16x8*>(kr + 32 * S::KPAD + c * 16);
          sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0f, qf[0][c], sc[0], 0, 0, 0);
          sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1f, qf[0][c], sc[1], 0, 0, 0);
        }
      } else if (act[0]) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 k0f = *reinterpret_cast<const bf16x8*>(kr + c * 16);
          sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0f, qf[0][c], sc[0], 0, 0, 0);
        }
      }
      bf16x8 pf[2][2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
        if (!MASKED || act[sub]) softmax32(sc[sub], 0, kt * KT + sub * 32, msk[sub], pf[sub]);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        if (MASKED && !act[sub]) continue;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
                vl_s + (db * 32 + krow_l) * S::VPAD + sub * 32 + kb * 16 + half * 8);
            o[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[sub][kb], o[0][db], 0, 0, 0);
          }
      }
    } else {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int k0 = kt * KT + sub * 32;
        bool act[R];
        bool msk[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const int qlo = c0 + t0 + rb_t[j];         // smallest query position of the row-block
          act[j] = MASKED ? (rb_ok[j] && k0 <= qlo + 31) : true;
          msk[j] = MASKED && k0 + 31 > qlo;
        }
        f32x16 sc[R];
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[j][i] = 0.f;
        const uint16_t* kr = kl_s + (sub * 32 + krow_l) * S::KPAD + half * 8;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kr + c * 16);
#pragma unroll
          for (int j = 0; j < R; ++j)
            if (act[j]) sc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[j][c], sc[j], 0, 0, 0);
        }
        bf16x8 pf[R][2];
#pragma unroll
        for (int j = 0; j < R; ++j)
          if (act[j]) softmax32(sc[j], j, k0, msk[j], pf[j]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
                vl_s + (db * 32 + krow_l) * S::VPAD + sub * 32 + kb * 16 + half * 8);
#pragma unroll
            for (int j = 0; j < R; ++j)
              if (act[j]) o[j][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[j][kb], o[j][db], 0, 0, 0);
          }
      }
    }
  };

  for (pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[j][db][i] = 0.f;
      l_run[j] = 0.f;
    }
    ovf = false;
    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int kt = 0; kt < ntk; ++kt) {
      const bool more = kt + 1 < ntk;
      if (more) load_tile(kt + 1);
      const uint16_t* kl_s = smem + (kt & 1) * S::BUF;
      const uint16_t* vl_s = kl_s + S::K_ELEMS;
      // tiles wholly at or below every row-block's smallest query position need
      // neither masks nor activity checks
      if (kt * KT + KT - 1 <= c0 + t0 && all_ok) {
        compute_tile(kl_s, vl_s, kt, std::integral_constant<bool, false>());
      } else {
        compute_tile(kl_s, vl_s, kt, std::integral_constant<bool, true>());
      }
      if (more) store_tile((kt + 1) & 1);
      __syncthreads();
    }
    // does any lane of the workgroup need a second pass?
    if (threadIdx.x == 0) redo = 0;
    __syncthreads();
    if (__any(ovf) && lane == 0) redo = 1;
    __syncthreads();
    if (!redo) break;
#pragma unroll
    for (int j = 0; j < R; ++j) m_ref[j] = m_seen[j];
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < R; ++j) {
    const float l_tot = l_run[j] + __shfl_xor(l_run[j], 32);
    const float inv = 1.f / l_tot;
    if (rb_ok[j] && rb_t[j] + col < qn) {
      uint16_t* orow = static_cast<uint16_t*>(a.O) + b * a.o_s0 + static_cast<int64_t>(rb_h[j]) * a.o_s1 +
                       static_cast<int64_t>(r0 + t0 + rb_t[j] + col) * a.o_s2;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = pack_bf16x2(o[j][db][kb * 8 + 2 * e] * inv, o[j][db][kb * 8 + 2 * e + 1] * inv);
          *reinterpret_cast<u32x4*>(orow + db * 32 + kb * 16 + half * 8) = w;
        }
    }
  }
}

// Heads per workgroup (Gc, dividing G) and 32-token blocks per workgroup (TB)
// with Gc * TB = 4 * R and TB >= GQA_PREFILL_MIN_TB (two 32-token blocks:
// 64-token query tiles match the 64-key tiles, which keeps the diagonal's
// masked work small): three row-blocks per wave when the group size allows,
// else two, else one.
struct PrefillShape {
  int Gc, TB, R;
};

#ifndef GQA_PREFILL_MAX_R
#define GQA_PREFILL_MAX_R 1
#endif

#ifndef GQA_PREFILL_MIN_TB
#define GQA_PREFILL_MIN_TB 2
#endif

static PrefillShape prefill_shape(int G) {
  for (int R = GQA_PREFILL_MAX_R; R >= 1; --R)
    for (int Gc = G; Gc >= 1; --Gc)
      if (G % Gc == 0 && (4 * R) % Gc == 0 && 4 * R / Gc >= GQA_PREFILL_MIN_TB) return {Gc, 4 * R / Gc, R};
  return {1, 4, 1};
}

hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const PrefillShape ps = prefill_shape(G);
  const int Tq = 32 * ps.TB;
  dim3 grid(a.Hkv * (G / ps.Gc), a.nseq, (a.n_rect + Tq - 1) / Tq);
  dim3 block(256);
#define GQA_LAUNCH(DD, RR) hipLaunchKernelGGL((prefill_bf16_kernel<DD, RR>), grid, block, 0, s, a, ps.Gc, ps.TB)
  if (a.d == 128) {
    if (ps.R == 3) GQA_LAUNCH(128, 3);
    else if (ps.R == 2) GQA_LAUNCH(128, 2);
    else GQA_LAUNCH(128, 1);
  } else {
    if (ps.R == 3) GQA_LAUNCH(64, 3);
    else if (ps.R == 2) GQA_LAUNCH(64, 2);
    else GQA_LAUNCH(64, 1);
  }
#undef GQA_LAUNCH
  return hipGetLastError();
}

}  // namespace gqa
