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
//    its query heads, sequence, 32*TB query tokens) with Gc*TB = 4: each wave
//    owns one row-block of 32 queries of one head, and every K/V tile staged
//    in LDS serves all Gc query heads of the group (the head map is an index;
//    the cache is never replicated).  Two workgroups share a CU, so each SIMD
//    runs two waves whose matrix-core and vector work interleave;
//  * 64-key K/V tiles (four pages) go from HBM straight into LDS with 16-byte
//    buffer loads (no staging registers, no per-tile address arithmetic: wave
//    w loads page w of the tile, the page offset is a scalar and every lane's
//    offset inside the page is fixed).  The LDS layouts are page-major and put
//    the 16 lanes of one read on 16 consecutive 16-byte chunks, so matrix-core
//    operand reads are free of bank conflicts;
//  * S^T = K q^T on v_mfma_f32_32x32x16_bf16 with keys as rows, so each lane
//    owns one query column; K rows are fed in a fixed permutation that makes
//    the score accumulator the B operand of O^T += V^T P^T as it stands, and
//    V pages are stored d-major so V^T operands are plain 16-byte reads;
//  * software pipeline: K runs one tile ahead of V, so while the softmax of
//    tile j runs on the vector unit the scores of tile j+1 run on the matrix
//    core; loads of K(j+2) and V(j+1) are in flight during tile j, and one
//    barrier per tile retires them;
//  * softmax in base 2 against a fixed reference per query row: the maximum
//    of the row's first 32 keys (key 0 is visible to every query, so the
//    reference is finite and a masked key never meets (-inf) - (-inf)).  The
//    loop keeps no running maximum and never rescales; the probabilities are
//    rounded to bf16 once, and their row sums are taken from those bf16 values
//    with dot2 instructions.  A row whose sum passes 2^64 (some score beyond
//    the reference by more than 2^64 in probability) or stays below 1/2 (no
//    visible key at the reference) makes the workgroup find the exact row
//    maxima in a score-only pass and run again against them, which can
//    neither overflow nor underflow;
//  * key tiles wholly in the future of the workgroup are never loaded;
//    masking by select happens only on tiles that cross the diagonal;
//  * value slots at or beyond the written length are zeroed in LDS by the
//    wave that loaded them, so stale or poisoned cache memory never meets a
//    zero weight (0 * NaN); stale keys only reach masked scores;
//  * workgroups are dispatched heaviest (last) query tile first, kv head
//    fastest, so with 8 kv heads workgroup i lands on XCD i % 8 = its kv head
//    and each XCD's L2 serves one head's keys and values.
#include <algorithm>

#include "common.hpp"
#include "device.hpp"

namespace gqa {

namespace {

constexpr int KT = 64;                 // keys per tile (four 16-slot pages)
#ifndef GQA_PF_LAK
#define GQA_PF_LAK 2
#endif
#ifndef GQA_PF_LAV
#define GQA_PF_LAV 3
#endif
constexpr int LAK = GQA_PF_LAK;        // score products a key operand read runs ahead
constexpr int LAV = GQA_PF_LAV;        // P.V products a value operand read runs ahead

// Swaps bits 2 and 3 (an involution).  MFMA row r is fed key (or d-row)
// perm32(r), which keeps the accumulator of rows 8*(i/4) + 4*half + i%4 equal
// to keys 16*(i/8) + 8*half + i%8.
__device__ __forceinline__ int perm32(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Buffer descriptor of a byte range (reads past num_records return zero).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return i32x4{static_cast<int>(p), static_cast<int>((p >> 32) & 0xffff), static_cast<int>(bytes), 0x00020000};
}

// 16 bytes per lane from buffer r at byte (voff + soff) into LDS byte
// lds_addr + 16*lane.  Written as one instruction so that the compiler does
// not order LDS reads of other buffers behind these loads; the caller waits
// (s_waitcnt vmcnt) and synchronises before the data is read.
__device__ __forceinline__ void dma16(i32x4 r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(r), "s"(soff));
}

// Keeps the computation of x at this point of the program: passes the value
// through an empty statement the compiler cannot move or look into.
template <typename T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// s_waitcnt immediate that waits for vector-memory count <= n only.
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Scalar 32-bit load of base[byte_off/4], issued without a wait: the value
// may be used only after sload_wait on it.
__device__ __forceinline__ int sload(const int32_t* base, uint32_t byte_off) {
  int v;
  asm volatile("s_load_dword %0, %1, %2" : "=s"(v) : "s"(base), "s"(byte_off));
  return v;
}
// Waits for outstanding scalar loads; the values pass through the statement
// so that no use of them can be placed before it.
__device__ __forceinline__ void sload_wait(int& a, int& b) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+s"(a), "+s"(b));
}

}  // namespace

template <int D, bool WIN>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(AttnArgs a, int Gc, int TB) {
  constexpr int NC = D / 16;           // k-steps of the score product
  constexpr int NDB = D / 32;          // 32-row blocks of the output
  constexpr int PCH = 2 * D;           // 16-byte chunks of one (page, kv head) of K or of V
  constexpr int NI = PCH / 64;         // buffer-to-LDS loads per wave per tile, for K and for V
  constexpr int TEL = KT * D;          // elements of a K or V tile
  __shared__ __attribute__((aligned(1024))) uint16_t smem[4 * TEL];   // K tiles 0, 1; V tiles 0, 1

  const int G = a.Hq / a.Hkv;
  const int hc = blockIdx.x / a.Hkv;
  const int g = blockIdx.x - hc * a.Hkv;
  const int b = blockIdx.y;
  const int tile = gridDim.z - 1 - blockIdx.z;
  const int Tq = 32 * TB;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int col = lane & 31;

  const int rw = a.meta.row[b];
  const int seq = a.meta.seq[rw];
  const int c0 = a.meta.start[b];
  const int nb = a.meta.count[b];
  const int r0 = a.meta.row0[b];
  const int total = a.meta.total[rw];
  const int br = a.meta.brow[rw];      // batch row of Q and O
  const int zlo = a.meta.zlo[b], zhi = a.meta.zhi[b];
  const int h0 = g * G + hc * Gc;      // first query head of this workgroup

  // padding rows of this entry's share [zlo, zhi) of the rectangle -> 0, Tq
  // rows per query tile counted from zlo (after every page-table read, so
  // those reads may use the scalar cache)
  auto zero_padding = [&]() {
    const int rlo = zlo + tile * Tq;
    const int rhi = min(zhi, rlo + Tq);
    const int per_row = D / 8;
    for (int idx = threadIdx.x; idx < Gc * Tq * per_row; idx += 256) {
      const int hh = idx / (Tq * per_row);
      const int rem = idx - hh * Tq * per_row;
      const int rr = rlo + rem / per_row;
      const int ch = rem % per_row;
      if (rr >= zlo && rr < rhi && (rr < r0 || rr >= r0 + nb)) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        uint16_t* op = static_cast<uint16_t*>(a.O) + br * a.o_s0 + static_cast<int64_t>(h0 + hh) * a.o_s1 +
                       static_cast<int64_t>(rr) * a.o_s2 + ch * 8;
        *reinterpret_cast<u32x4*>(op) = z;
      }
    }
  };

  const int t0 = tile * Tq;
  if (t0 >= nb) {
    zero_padding();
    return;
  }
  const int qn = min(Tq, nb - t0);

  // this wave's row-block: head, first token, validity; the lane's query
  const int rb_h = h0 + wave / TB;
  const int rb_t = (wave % TB) * 32;
  const bool q_ok = rb_t + col < qn;
  const int qpos = c0 + t0 + rb_t + col;

  // rotated queries as B operands: lane holds dims 16c + 8*half + 0..7 of its
  // query (loaded once the first key/value tiles are in flight)
  bf16x8 qf[NC];
  const int kv_end = c0 + t0 + qn;            // keys [0, kv_end) can be visible
  // sliding window: key tiles wholly before the first query's window are never
  // read; tile j of this workgroup is key tile kt0 + j
  const int kt0 = WIN ? max(0, c0 + t0 - a.window + 1) / KT : 0;
  const int ntk = (kv_end + KT - 1) / KT - kt0;
  const int last_page = (total - 1) >> 4;
  const int32_t* trow = a.table + static_cast<int64_t>(seq) * a.table_w;
  const int Hkv = a.Hkv;
  const float sl2 = a.scale_log2;
  const i32x4 krs = make_rsrc(a.k_pool, a.pool_bytes);
  const i32x4 vrs = make_rsrc(a.v_pool, a.pool_bytes);

  // LDS: K tiles at [0, 2*TB_), V tiles at [2*TB_, 4*TB_) bytes
  constexpr uint32_t TB_ = TEL * 2;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)(smem)));
  const uint16_t* ks[2] = {smem, smem + TEL};
  const uint16_t* vs[2] = {smem + 2 * TEL, smem + 3 * TEL};

  // ---- HBM -> LDS.  Wave w loads page w of a tile.  K: LDS chunk
  // (page, cc, perm32(key)) holds dims 8cc..8cc+7 of the page's key; V: LDS
  // chunk (page, h8, perm32(d-row)) holds slots 8*h8..8*h8+7 of that d-row.
  // The lane offset inside the page is fixed; the page and the instruction's
  // share of it go in the scalar offset.
  const uint32_t kvo = static_cast<uint32_t>(perm32(lane & 15) * (2 * D) + (lane >> 4) * 16);
  const uint32_t vvo = static_cast<uint32_t>(perm32(lane) * 32);
  // page-table entry of this wave's page of tile kt: a scalar load whose
  // wait is placed by the caller (sload_wait), so it never waits on the
  // buffer-to-LDS loads in flight
  auto page_id = [&](int kt) -> int {
    int lp = min((kt0 + kt) * 4 + wave, last_page);
    if constexpr (WIN) lp = __builtin_amdgcn_readfirstlane(lp % a.table_w);   // a windowed cache is a ring
    return sload(trow, static_cast<uint32_t>(lp) * 4u);
  };
  auto page_off = [&](int phys) -> uint32_t {
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(phys) * Hkv + g) * static_cast<uint32_t>(32 * D);
  };
  auto issue_k = [&](int phys, int buf) {
    const uint32_t so = page_off(phys);
    const uint32_t dst = lds0 + buf * TB_ + wave * (PCH * 16);
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(krs, dst + i * 1024, kvo, so + i * 64);
  };
  auto issue_v = [&](int phys, int buf) {
    const uint32_t so = page_off(phys);
    const uint32_t dst = lds0 + (2 + buf) * TB_ + wave * (PCH * 16);
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(vrs, dst + i * 1024, vvo, so + ((i * 64) % D) * 32 + ((i * 64) / D) * 16);
  };
  // zero the value slots >= total of this wave's page of tile kt (after its loads landed)
  auto fix_v = [&](int kt, int buf) {
    const int s0 = (kt * 4 + wave) * 16;
    if (s0 + 16 <= total) return;
    uint16_t* reg = smem + (2 + buf) * TEL + wave * PCH * 8;
#pragma unroll
    for (int r = 0; r < NI; ++r) {
      const int q = r * 64 + lane;
      const int slot = s0 + (q / D) * 8;
      u32x4 w = *reinterpret_cast<u32x4*>(reg + q * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t keep_lo = (slot + 2 * e < total) ? 0x0000ffffu : 0u;
        const uint32_t keep_hi = (slot + 2 * e + 1 < total) ? 0xffff0000u : 0u;
        w[e] &= (keep_lo | keep_hi);
      }
      *reinterpret_cast<u32x4*>(reg + q * 8) = w;
    }
  };

  // LDS read offsets (elements) of this lane's MFMA operands
  const int kread = ((col >> 4) * PCH + half * 16 + (col & 15)) * 8;
  const int vread = (half * D + col) * 8;

  auto qk = [&](const uint16_t* kb, f32x16 (&s)[2]) {
    const uint16_t* kr = kb + kread;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kr + c * 256);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(kr + 2 * PCH * 8 + c * 256);
      if (c == 0) {
        const f32x16 z = {};
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[0], z, 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[0], z, 0, 0, 0);
      } else {
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[c], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[c], s[1], 0, 0, 0);
      }
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float l0 = 0.f, l1 = 0.f, mneg;
  const bf16x2 ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;

  // Two softmax elements i, i+1 (i even) of a 32-key sub-tile whose first key
  // is k0: probabilities against the row reference, rounded to bf16 into the
  // B operand pf (8 elements per 16-key half), row sum of the rounded values.
  auto sm2 = [&](const f32x16& s, int i, int k0, bf16x8& pf, float& l, auto masked) {
    float x0 = s[i], x1 = s[i + 1];
    if constexpr (decltype(masked)::value) {
      const int lim = qpos - k0 - 8 * half;     // key k0 + 16*(i/8) + 8*half + i%8 visible iff offset <= lim
      if (16 * (i >> 3) + (i & 7) > lim) x0 = -INFINITY;
      if (16 * (i >> 3) + (i & 7) + 1 > lim) x1 = -INFINITY;
      if constexpr (WIN) {                      // and offset > lim - window
        if (16 * (i >> 3) + (i & 7) <= lim - a.window) x0 = -INFINITY;
        if (16 * (i >> 3) + (i & 7) + 1 <= lim - a.window) x1 = -INFINITY;
      }
    }
    const bf16x2 p = {static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(x0, sl2, mneg))),
                      static_cast<__bf16>(__builtin_amdgcn_exp2f(fmaf(x1, sl2, mneg)))};
    l = __builtin_amdgcn_fdot2_f32_bf16(p, ones, l, false);
    pf[i & 7] = p[0];
    pf[(i & 7) + 1] = p[1];
  };
  auto kfrag = [&](const uint16_t* kb, int c, int sub) {
    return *reinterpret_cast<const bf16x8*>(kb + kread + sub * 2 * PCH * 8 + c * 256);
  };
  auto vfrag = [&](const uint16_t* vb, int sub, int kb, int db) {
    return *reinterpret_cast<const bf16x8*>(vb + vread + ((sub * 2 + kb) * PCH + db * 32) * 8);
  };

  // One tile of the pipeline in two phases, their order fixed by scheduling
  // fences.  Phase A: the score products of tile j+1 (when NEXT; K in kb,
  // into nxt) carry the softmax of sub-tile 0 of tile j (scores in cur).
  // Phase B: P.V of tile j (V in vb), whose first half carries the softmax of
  // sub-tile 1.  Operand reads run one (K) or two (V) products ahead.
  auto phase_a = [&](f32x16 (&cur)[2], f32x16 (&nxt)[2], const uint16_t* kb, int kbase, bf16x8 (&pf)[2][2],
                     auto masked, auto next) {
    if constexpr (decltype(next)::value) {
      bf16x8 kq[NC][2];
#pragma unroll
      for (int c = 0; c < LAK && c < NC; ++c) {
        kq[c][0] = kfrag(kb, c, 0);
        kq[c][1] = kfrag(kb, c, 1);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (c + LAK < NC) {
          kq[c + LAK][0] = kfrag(kb, c + LAK, 0);
          kq[c + LAK][1] = kfrag(kb, c + LAK, 1);
        }
        if (c == 0) {
          const f32x16 z = {};
          nxt[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[0][0], qf[0], z, 0, 0, 0);
          nxt[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[0][1], qf[0], z, 0, 0, 0);
        } else {
          nxt[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[c][0], qf[c], nxt[0], 0, 0, 0);
          nxt[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[c][1], qf[c], nxt[1], 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < 16 / NC; t += 2) {
          const int i = c * (16 / NC) + t;
          sm2(cur[0], i, kbase, pf[0][i >> 3], l0, masked);
        }
        pin(pf[0][(c * (16 / NC)) >> 3]);
        pin(l0);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; i += 2) sm2(cur[0], i, kbase, pf[0][i >> 3], l0, masked);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto phase_b = [&](f32x16 (&cur)[2], const uint16_t* vb, int kbase, bf16x8 (&pf)[2][2], auto masked) {
    constexpr int NU = 4 * NDB;
    auto vfrag_u = [&](int u) { return vfrag(vb, u / (2 * NDB), (u / NDB) & 1, u % NDB); };
    bf16x8 vq[NU];
#pragma unroll
    for (int u = 0; u < LAV && u < NU; ++u) vq[u] = vfrag_u(u);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int sub = u / (2 * NDB), kk = (u / NDB) & 1, db = u % NDB;
      if (u + LAV < NU) vq[u + LAV] = vfrag_u(u + LAV);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vq[u], pf[sub][kk], o[db], 0, 0, 0);
      if (u < 2 * NDB) {
#pragma unroll
        for (int t = 0; t < 16 / (2 * NDB); t += 2) {
          const int i = u * (16 / (2 * NDB)) + t;
          sm2(cur[1], i, kbase + 32, pf[1][i >> 3], l1, masked);
        }
        pin(pf[1][(u * (16 / (2 * NDB))) >> 3]);
        pin(l1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Wait until at most n of this wave's buffer-to-LDS loads are in flight
  // (they complete in issue order); n is 0, NI or 2*NI.
  auto wait_vm = [&](int n) {
    if (n >= 2 * NI) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NI));
    else if (n >= NI) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NI));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  };

  // Step j (P = j & 1).  On entry K(j+1) sits in K buffer 1-P, V(j) is in
  // flight or landed in V buffer P, K(j+2) is in flight to K buffer P, and
  // the scores of tile j are in cur.  V(j+1) is issued at the start (into V
  // buffer 1-P, free since P.V of tile j-1), K(j+3) after the mid-step
  // barrier (into K buffer 1-P, free once every wave has scored tile j+1), so
  // each load has about one and a half steps to land.  MODE any = false: a
  // tile wholly visible to every query of the workgroup, with a next tile.
  int pg_v = 0, pg_k = 0;                    // pages of V(j+1) and K(j+3) for step j
  auto step = [&](int j, f32x16 (&cur)[2], f32x16 (&nxt)[2], auto parity, auto any) {
    constexpr int P = decltype(parity)::value ? 1 : 0;
    const bool has_next = j + 1 < ntk;
    if (has_next) issue_v(pg_v, 1 - P);
    const int nv = page_id(j + 2), nk = page_id(j + 4);
    const int kbase = (kt0 + j) * KT;
    bf16x8 pf[2][2];
    if constexpr (!decltype(any)::value) {
      phase_a(cur, nxt, ks[1 - P], kbase, pf, F_(), T_());
    } else {
      if (has_next) phase_a(cur, nxt, ks[1 - P], kbase, pf, T_(), T_());
      else phase_a(cur, nxt, ks[1 - P], kbase, pf, T_(), F_());
    }
    // V(j) must have landed; K(j+2) and V(j+1) may still be in flight
    wait_vm((j + 2 < ntk ? NI : 0) + (has_next ? NI : 0));
    fix_v(kt0 + j, P);
    __syncthreads();
    if (j + 3 < ntk) issue_k(pg_k, 1 - P);
    if constexpr (!decltype(any)::value) phase_b(cur, vs[P], kbase, pf, F_());
    else phase_b(cur, vs[P], kbase, pf, T_());
    // K(j+2) must have landed; V(j+1) and K(j+3) may still be in flight
    wait_vm((has_next ? NI : 0) + (j + 3 < ntk ? NI : 0));
    pg_v = nv;
    pg_k = nk;
    sload_wait(pg_v, pg_k);
    __syncthreads();
  };

  f32x16 sA[2], sB[2];
  {
    int p0 = page_id(0), p1 = page_id(1);
    sload_wait(p0, p1);
    issue_k(p0, 0);
    issue_v(p0, 0);
    if (ntk > 1) issue_k(p1, 1);
    pg_v = page_id(1);
    int p2 = page_id(2);
    pg_k = page_id(3);
    {
      // every lane loads a valid row (padding lanes reuse the last valid one
      // and are zeroed), so all query and rotation-table loads issue together
      const int tq = min(rb_t + col, qn - 1);
      const uint16_t* qrow = static_cast<const uint16_t*>(a.Q) + br * a.q_s0 + static_cast<int64_t>(rb_h) * a.q_s1 +
                             static_cast<int64_t>(r0 + t0 + tq) * a.q_s2;
      u32x4 w[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) w[c] = *reinterpret_cast<const u32x4*>(qrow + c * 16 + half * 8);
      f32x4 cs[NC / 2][4];                   // (cos, sin) of pairs 16c + 8*half + 0..7
      if (a.rope) {
        // chunk-major copy of the table: chunk 8c + 4*half + q4 of this lane's
        // position; the 32 lanes of a half read 32 consecutive positions of one
        // chunk, 512 contiguous bytes
        const float* rcol = a.rope_t + static_cast<int64_t>(c0 + t0 + tq) * 4;
#pragma unroll
        for (int c = 0; c < NC / 2; ++c)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            cs[c][q4] = *reinterpret_cast<const f32x4*>(
                rcol + static_cast<int64_t>(8 * c + 4 * half + q4) * a.rope_rows * 4);
      }
      float x[NC][8];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t v = q_ok ? w[c][e] : 0u;
          x[c][2 * e] = __uint_as_float(v << 16);
          x[c][2 * e + 1] = __uint_as_float(v & 0xffff0000u);
        }
      if (a.rope) {
#pragma unroll
        for (int c = 0; c < NC / 2; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float lo, hi;
            rotate_pair(x[c][e], x[c + NC / 2][e], cs[c][e / 2][(e % 2) * 2], cs[c][e / 2][(e % 2) * 2 + 1], lo,
                        hi);
            x[c][e] = lo;
            x[c + NC / 2][e] = hi;
          }
      }
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[c][e] = static_cast<__bf16>(x[c][e]);
    }
    sload_wait(pg_v, p2);
    sload_wait(pg_k, p2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    qk(ks[0], sA);
    float mx = -INFINITY;
    if constexpr (!WIN) {
      // reference: maximum of the row's visible keys among keys 0..31
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 16 * (i >> 3) + 8 * half + (i & 7);
        mx = fmaxf(mx, key <= qpos ? sA[0][i] : -INFINITY);
      }
    } else {
      // reference: maximum of the row's visible keys among the key tiles that
      // hold its first visible key.  A row's window starts at most Tq - 1
      // keys after the first row's, so with 64-token query tiles the first
      // two tiles read hold every row's first visible key, and with 128-token
      // tiles the first three do (the third is taken below when some row needs it)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt0 * KT + sub * 32 + 16 * (i >> 3) + 8 * half + (i & 7);
          mx = fmaxf(mx, key <= qpos && key > qpos - a.window ? sA[sub][i] : -INFINITY);
        }
      if (ntk > 1) {
        qk(ks[1], sB);                       // K(1) has landed; step 0 computes these scores again
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = (kt0 + 1) * KT + sub * 32 + 16 * (i >> 3) + 8 * half + (i & 7);
            mx = fmaxf(mx, key <= qpos && key > qpos - a.window ? sB[sub][i] : -INFINITY);
          }
      }
    }
    __syncthreads();                         // K(0) is read by every wave before K(2) replaces it
    if (ntk > 2) issue_k(p2, 0);
    if constexpr (WIN) {
      // the last row's window starts at or past key tile kt0 + 2: wait for
      // K(2) and take its visible keys too (step 0 overwrites sB again)
      if (ntk > 2 && c0 + t0 + qn - a.window >= (kt0 + 2) * KT) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        qk(ks[0], sB);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = (kt0 + 2) * KT + sub * 32 + 16 * (i >> 3) + 8 * half + (i & 7);
            mx = fmaxf(mx, key <= qpos && key > qpos - a.window ? sB[sub][i] : -INFINITY);
          }
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (WIN && mx == -INFINITY) mx = 0.f;    // padding lanes only
    mneg = -(mx * sl2);
  }
  // leading tiles wholly visible to the whole workgroup (each with a next
  // tile) in pairs, then the rest with masks
  const int nfull = min((c0 + t0 + 1) / KT - kt0, ntk - 1);
  int j = 0;
  if constexpr (WIN) {
    // one step with the buffers and parity of its index
    auto one = [&](int jj, auto masked) {
      if (jj & 1) step(jj, sB, sA, T_(), masked);
      else step(jj, sA, sB, F_(), masked);
    };
    // leading tiles that reach below the last row's window start need masks
    const int ws_last = max(0, c0 + t0 + qn - a.window);
    const int jlo = min((ws_last + KT - 1) / KT - kt0, ntk);
    for (; j + 2 <= jlo; j += 2) {
      step(j, sA, sB, F_(), T_());
      step(j + 1, sB, sA, T_(), T_());
    }
    if (j < jlo) {
      step(j, sA, sB, F_(), T_());
      ++j;
    }
    if ((j & 1) && j < nfull) {
      one(j, F_());
      ++j;
    }
    for (; j + 2 <= nfull; j += 2) {
      step(j, sA, sB, F_(), F_());
      step(j + 1, sB, sA, T_(), F_());
    }
    if ((j & 1) && j < ntk) {
      one(j, T_());
      ++j;
    }
  } else {
    for (; j + 2 <= nfull; j += 2) {
      step(j, sA, sB, F_(), F_());
      step(j + 1, sB, sA, T_(), F_());
    }
  }
  for (; j < ntk; j += 2) {
    step(j, sA, sB, F_(), T_());
    if (j + 1 < ntk) step(j + 1, sB, sA, T_(), T_());
  }

  // A row whose sum passed 2^64 (or is not finite) had a score far above its
  // reference: find the exact row maxima (scores only) and run once more,
  // one tile at a time, against them.  A reference taken from one of the
  // row's visible keys gives that key the probability 1, so a sum below 1/2
  // means the reference missed the row's keys: the same pass handles it.
  float l = l0 + l1;
  float l_tot = l + __shfl_xor(l, 32);
  if (__syncthreads_or(q_ok && !(l_tot >= 0.5f && l_tot <= 0x1p64f))) {
    float m = -INFINITY;
    for (int kt = 0; kt < ntk; ++kt) {
      int pid = page_id(kt), unused = 0;
      sload_wait(pid, unused);
      issue_k(pid, 0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      qk(ks[0], sA);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = (kt0 + kt) * KT + sub * 32 + 16 * (i >> 3) + 8 * half + (i & 7);
          m = fmaxf(m, key <= qpos && (!WIN || key > qpos - a.window) ? sA[sub][i] : -INFINITY);
        }
      __syncthreads();
    }
    m = fmaxf(m, __shfl_xor(m, 32));
    mneg = -(m * sl2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    l0 = 0.f;
    l1 = 0.f;
    for (int kt = 0; kt < ntk; ++kt) {
      int pid = page_id(kt), unused = 0;
      sload_wait(pid, unused);
      issue_k(pid, 0);
      issue_v(pid, 0);
      __builtin_amdgcn_s_waitcnt(0);
      fix_v(kt0 + kt, 0);
      __syncthreads();
      qk(ks[0], sA);
      bf16x8 pf[2][2];
      phase_a(sA, sB, ks[0], (kt0 + kt) * KT, pf, T_(), F_());
      phase_b(sA, vs[0], (kt0 + kt) * KT, pf, T_());
      __syncthreads();
    }
    l = l0 + l1;
    l_tot = l + __shfl_xor(l, 32);
  }

  const float inv = 1.f / l_tot;
  if (q_ok) {
    uint16_t* orow = static_cast<uint16_t*>(a.O) + br * a.o_s0 + static_cast<int64_t>(rb_h) * a.o_s1 +
                     static_cast<int64_t>(r0 + t0 + rb_t + col) * a.o_s2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = static_cast<__bf16>(o[db][kb * 8 + e] * inv);
        *reinterpret_cast<bf16x8*>(orow + db * 32 + kb * 16 + half * 8) = w;
      }
  }
  zero_padding();
}

// Heads per workgroup (Gc, dividing G) and 32-token blocks per workgroup (TB)
// with Gc * TB = 4 (one row-block per wave) and TB >= 2: 64-token query tiles
// match the 64-key tiles, which keeps the diagonal's masked work small.  When
// 64-token tiles would leave more than an eighth of their rows idle (short or
// ragged runs, masks with holes) and 4 divides G, 32-token tiles of four heads
// are used instead.
struct PrefillShape {
  int Gc, TB;
};

static PrefillShape prefill_shape(int G, int64_t idle64, int64_t rows64) {
  if (G % 4 == 0 && idle64 * 8 > rows64) return {4, 1};
  for (int Gc = 2; Gc >= 1; --Gc)
    if (G % Gc == 0) return {Gc, 4 / Gc};
  return {1, 4};
}

hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  int64_t rows64 = 0, idle64 = 0;             // rows of 64-token tiles, and those without a query
  for (int j = 0; j < a.nseq; ++j) {
    const int64_t t64 = (a.meta.count[j] + 63) / 64 * 64;
    rows64 += t64;
    idle64 += t64 - a.meta.count[j];
  }
  const PrefillShape ps = prefill_shape(G, idle64, rows64);
  const int Tq = 32 * ps.TB;
  // query tiles: enough for the longest share of rows (its run and the padding
  // it zeroes), never more, so entries of short runs launch no idle tiles
  int rows = 1;
  for (int j = 0; j < a.nseq; ++j) rows = std::max(rows, a.meta.zhi[j] - a.meta.zlo[j]);
  dim3 grid(a.Hkv * (G / ps.Gc), a.nseq, (rows + Tq - 1) / Tq);
  dim3 block(256);
  if (a.window) {
    if (a.d == 128)
      hipLaunchKernelGGL((prefill_bf16_kernel<128, true>), grid, block, 0, s, a, ps.Gc, ps.TB);
    else
      hipLaunchKernelGGL((prefill_bf16_kernel<64, true>), grid, block, 0, s, a, ps.Gc, ps.TB);
  } else if (a.d == 128) {
    hipLaunchKernelGGL((prefill_bf16_kernel<128, false>), grid, block, 0, s, a, ps.Gc, ps.TB);
  } else {
    hipLaunchKernelGGL((prefill_bf16_kernel<64, false>), grid, block, 0, s, a, ps.Gc, ps.TB);
  }
  return hipGetLastError();
}

}  // namespace gqa
