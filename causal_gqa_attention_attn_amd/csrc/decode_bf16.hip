// bfloat16 split-T attention over the paged cache for decode and short query
// chunks, one launch per layer.
//
// What it computes (page "模型执行：从 token 到 Prefill 与 Decode", prefill and
// decode shapes; page "KV Cache 与 Prefill/Decode 推理路径", single-token
// decode needs no mask): one new query per sequence, at position T-1, attends
// to all T cached slots of its KV head g(h) = floor(h*Hkv/Hq):
//   o[b,h] = sum_{j<T} softmax_j(<rot(q), k_used[g,j]>/sqrt(d)) v[g,j].
// More generally a sequence brings a run of `count` queries at positions
// start, start+1, ... (a verify chunk, or rows inside a cached sequence; page
// "Prefill：整层状态演化与 KV 建立", 2.3 causal mask): the query at position p
// attends to slots 0..p only.  Each (query token t, head h) pair is one matrix
// column c = t*G + h, with its own rotation row and causal limit; decode is the
// run of one.  Rectangular rows of o outside the run are written as 0.
// Optionally the same launch first appends the step's new token (slot T-1):
// its key is rotated with the query's rotation row (same position) and
// rounded to bf16, its value copied, both written to the cache and used
// straight from registers.
//
// How (memory-bound; every K/V byte is read from HBM once per step):
//  * one workgroup = (sequence, split of consecutive pages, kv head, up to 16
//    (token, head) columns of its group); its four waves take the split's pages in turn,
//    each with two pages in flight; the block-table entries, the query
//    and its rotation row are requested together before any is used;
//  * per two pages of a wave (one block of 32 keys): S^T[16 keys x 16
//    columns] = K q^T on v_mfma_f32_16x16x32_bf16 for each half of the block,
//    K rows loaded straight from the pages in an order that makes the two
//    score accumulators the B operand of O^T[d x heads] += V^T P^T, also on
//    v_mfma_f32_16x16x32_bf16, whose V^T operand is 8 consecutive slots of
//    one d-row of the d-major page: every K and V load is 16 bytes wide;
//  * online softmax in base 2 per column; the four waves, then the splits, are
//    combined with the log-sum-exp rule: with M = max_s m_s,
//    O = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M);
//  * split combine inside the launch, without atomics (same-address
//    device-scope atomics serialise across the chip's XCDs): every split
//    writes its (m, l, o) record with device-scope stores and then a ready flag
//    for each merger.  The mergers are the last (up to four) splits of the
//    (sequence, kv head, column chunk) - the highest workgroup indices of the group, so they
//    only wait on workgroups dispatched before them or on each other, and
//    there are never more of them than the chip holds at once.  Each polls its
//    flags with a bounded spin, combines its share of the output columns and
//    clears its own flag row for the next call.  A split writes the call's
//    epoch (a nonzero number the host changes from call to call) as its flag,
//    so a flag left by an earlier call that gave up never passes for a new
//    one; a merger that gives up writes NaN and sets the workspace's sticky
//    status word, which the host reads back as an error.
#include "common.hpp"
#include "device.hpp"

namespace gqa {

namespace {

#ifndef GQA_DECODE_BATCH
#define GQA_DECODE_BATCH 2                 // pages a wave keeps in flight
#endif
constexpr int kMergeBatch = 8;             // split records a merging thread loads at once
constexpr int kSc1 = 16;                   // buffer cache policy: sc1 (device-scope coherent)
constexpr int kBufferWord3 = 0x00020000;   // buffer resource word 3: raw 32-bit dword access

typedef float float2_t __attribute__((ext_vector_type(2)));

}  // namespace

// CHUNK: some sequence brings more than one query (or rectangular padding
// rows); WIN: the cache has a sliding window.  Plain decode takes neither, so
// its instructions carry no per-column position arithmetic.  In chunk mode a
// workgroup takes two 16-column chunks of its kv head, which share every K/V
// load.
// NEWP: some sequence's new token opens a page in this launch (a.new_page);
// launches without one take the variant that never looks at new_page.
template <int D, bool CHUNK, bool WIN, bool NEWP>
__global__ __launch_bounds__(256, 2) void decode_bf16_kernel(DecodeArgs a) {
  constexpr int NQ = D / 32;      // k-steps of the score product
  constexpr int NDB = D / 16;     // 16-row blocks of the output
  constexpr int NCH = CHUNK ? 2 : 1;   // 16-column chunks per workgroup
  __shared__ float red_m[4][16 * NCH];
  __shared__ float red_l[4][16 * NCH];
  __shared__ float red_o[4][16 * NCH][D + 4];
  __shared__ int s_ok;

  const int G = a.Hq / a.Hkv;
  const int hchunks = (a.ncol + 15) >> 4;           // 16-column chunks per kv head
  const int hgroups = (hchunks + NCH - 1) / NCH;    // workgroup rows per kv head
  const int gy = a.Hkv * hchunks;                   // (kv head, column chunk) rows of the split records
  // Chunks: blockIdx.x = (split, chunk group, kv head), kv head fastest: the
  // workgroups running at one time cover every kv head of the same few pages
  // (whole 32 KiB page rows of the pool), and the chunk groups of one (split,
  // kv head) run Hkv workgroups apart, on the same XCD (workgroup index mod 8)
  // when Hkv is a multiple of 8, so the later ones find the pages in its L2.
  // Plain decode: blockIdx.x = split, blockIdx.y = (kv head, column chunk),
  // which measured faster for a single long sequence.
  int g, hgr, gsplit;
  if constexpr (CHUNK) {
    g = blockIdx.x % a.Hkv;
    const int xr = blockIdx.x / a.Hkv;
    hgr = xr % hgroups;
    gsplit = xr / hgroups;
  } else {
    g = blockIdx.y / hchunks;
    hgr = blockIdx.y - g * hchunks;
    gsplit = blockIdx.x;
  }
  const int hcb0 = hgr * NCH;                       // first column chunk of this workgroup
  // this workgroup's sequence: the last b with split_off[b] <= gsplit (the
  // offsets increase strictly), found by binary lifting over the arguments
  int b = 0;
#pragma unroll
  for (int step = kMaxSeqPerLaunch / 2; step >= 1; step >>= 1)
    if (b + step < a.nseq && a.split_off[b + step] <= gsplit) b += step;
  const int split = gsplit - a.split_off[b];
  const int nsplit = a.split_off[b + 1] - a.split_off[b];
  const int seq = a.meta.seq[b];
  const int T = a.meta.total[b];
  const int start = a.meta.start[b];
  const int cnt = CHUNK ? a.meta.count[b] : 1;
  const int r0 = CHUNK ? a.meta.row0[b] : 0;
  const int br = a.meta.brow[b];           // batch row of q, o and the new token
  const int npages = (T + kPage - 1) / kPage;
  // sliding window: pages wholly before the first query's window are never read
  const int p_lo = WIN ? max(0, start - a.window + 1) / kPage : 0;
  const int p_begin = p_lo + split * a.pages_per_split;
  const int p_end = min(npages, p_begin + a.pages_per_split);

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;
  const int c16 = lane & 15;

  // padding rows of o (rectangular rows outside the sequence's query run) -> 0,
  // by the first split of the first chunk group of each kv head
  if (CHUNK && split == 0 && hgr == 0 && a.n_rect > cnt) {
    for (int idx = threadIdx.x; idx < G * a.n_rect * (D / 8); idx += 256) {
      const int hh = idx / (a.n_rect * (D / 8));
      const int rem = idx - hh * a.n_rect * (D / 8);
      const int rr = rem / (D / 8);
      const int ch = rem - rr * (D / 8);
      if ((rr < r0 || rr >= r0 + cnt) && rr >= a.meta.zlo[b] && rr < a.meta.zhi[b]) {
        uint16_t* op = static_cast<uint16_t*>(a.o) + br * a.o_s0 + static_cast<int64_t>(g * G + hh) * a.o_s1 +
                       static_cast<int64_t>(rr) * a.o_s2 + ch * 8;
        *reinterpret_cast<u32x4*>(op) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  // Columns of the matrix products are (query token t, head h) pairs, column
  // c = t*G + h; chunk ch of this workgroup holds columns 16*(hcb0+ch) + 0..15.
  int Gc[NCH];                                  // valid columns of each chunk for this sequence
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) Gc[ch] = min(16, cnt * G - (hcb0 + ch) * 16);
  if (Gc[0] <= 0) return;                       // (every split of the group returns here)
  const bool two = NCH > 1 && Gc[NCH - 1] > 0;  // the second chunk has columns
  bool hvalid[NCH];
  int hl[NCH], tl[NCH], qpos[NCH];              // this lane's column: head, token, position
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const int cl = (hcb0 + ch) * 16 + c16;
    hvalid[ch] = cl < cnt * G;
    const int clc = min(cl, cnt * G - 1);
    tl[ch] = CHUNK ? clc / G : 0;
    hl[ch] = clc - tl[ch] * G;
    qpos[ch] = start + tl[ch];                  // keys 0..qpos are visible
  }
  // o row of column c of chunk ch
  auto out_row = [&](int ch, int c) {
    const int col = (hcb0 + ch) * 16 + c;
    const int t = CHUNK ? col / G : 0;
    return static_cast<uint16_t*>(a.o) + br * a.o_s0 + static_cast<int64_t>(g * G + col - t * G) * a.o_s1 +
           static_cast<int64_t>(r0 + t) * a.o_s2;
  };

  uint16_t* kpool = static_cast<uint16_t*>(a.k_pool);
  uint16_t* vpool = static_cast<uint16_t*>(a.v_pool);
  const int32_t* trow = a.table + static_cast<int64_t>(seq) * a.table_w;
  auto tix = [&](int p) { return WIN ? p % a.table_w : p; };   // a windowed cache is a ring
  const int Hkv = a.Hkv;
  const float sl2 = a.scale_log2;

  // the step's new token (slot T-1) lives in the last page, so in the last split
  const bool owns_new = !CHUNK && a.k_new != nullptr && split == nsplit - 1;
  const int p_new = (T - 1) >> 4;
  const int r_new = (T - 1) & 15;
  // a page this call opens for the new token: its block-table entry is not on
  // the device yet; this launch reads the page from its arguments and writes
  // the entry for later calls (no other split reads that page)
  const int new_phys = NEWP && owns_new ? a.new_page[b] : -1;
  if (new_phys >= 0 && g == 0 && hgr == 0 && threadIdx.x == 0) a.table[static_cast<int64_t>(seq) * a.table_w + tix(p_new)] = new_phys;
  auto table_at = [&](int p) -> int64_t {
    const int64_t t = trow[tix(p)];                 // loaded either way: no branch around the load
    return new_phys >= 0 && p == p_new ? static_cast<int64_t>(new_phys) : t;
  };

  // Everything the first batch needs is requested before anything is used:
  // the block-table entries of this wave's pages, the queries, their rotation
  // rows and the new token.  Loads are unconditional (indices clamped to valid
  // rows) so the compiler issues them back to back.
  constexpr int kBatch = GQA_DECODE_BATCH;
  const int p_first = p_begin + wave;
  int64_t phys[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) phys[j] = table_at(min(p_first + 4 * j, p_end - 1));
  u32x4 qw[NCH][NQ];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + br * a.q_s0 +
                           static_cast<int64_t>(g * G + hl[ch]) * a.q_s1 + static_cast<int64_t>(r0 + tl[ch]) * a.q_s2;
#pragma unroll
    for (int c = 0; c < NQ; ++c) qw[ch][c] = *reinterpret_cast<const u32x4*>(qrow + c * 32 + grp * 8);
  }
  u32x4 kw[NQ];
  uint32_t vw[NDB];
  if (owns_new) {
    const uint16_t* krow = static_cast<const uint16_t*>(a.k_new) + br * a.kn_s0 + static_cast<int64_t>(g) * a.kn_s1;
    const uint16_t* vrow = static_cast<const uint16_t*>(a.v_new) + br * a.vn_s0 + static_cast<int64_t>(g) * a.vn_s1;
#pragma unroll
    for (int c = 0; c < NQ; ++c) kw[c] = *reinterpret_cast<const u32x4*>(krow + c * 32 + grp * 8);
#pragma unroll
    for (int db = 0; db < NDB; ++db) vw[db] = vrow[db * 16 + c16];
  }
  float cs[NCH][NQ / 2][8][2];
  if (a.rope) {
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const float* rrow = a.rope + static_cast<int64_t>(qpos[ch]) * D;
#pragma unroll
      for (int c = 0; c < NQ / 2; ++c) {
        const float4* r4 = reinterpret_cast<const float4*>(rrow + 2 * (c * 32 + grp * 8));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float4 v = r4[e];
          cs[ch][c][2 * e][0] = v.x;
          cs[ch][c][2 * e][1] = v.y;
          cs[ch][c][2 * e + 1][0] = v.z;
          cs[ch][c][2 * e + 1][1] = v.w;
        }
      }
    }
  }
  // A batch is the wave's two pages p0 and p0 + 4, taken as one block of 32
  // keys.  Key order inside the block (the k index of the P.V product): k =
  // 8*g + e is slot 8*(g%2) + e of page g/2 (g = 0..3), so that a lane's V^T
  // operand is 8 consecutive slots of one d-row of one page, a 16-byte load.
  // The score products take K rows in the matching order (row r of half-block
  // v is slot 8*((r/4)%2) + 4v + r%4 of page r/8), which leaves in lane
  // (column, g) the scores of keys k = 8g + 4v + 0..3: elements 4v..4v+3 of
  // its B operand of the P.V product, as they stand.
  static_assert(kBatch == 2, "a batch is two pages");
  const int kslot0 = 8 * ((c16 >> 2) & 1) + (c16 & 3);   // K row slot of half-block 0 (+4 for half-block 1)
  auto load_pages = [&](const int64_t* ph, bf16x8 (*kf)[NQ], u32x4* vf) {
    const int64_t kph = c16 < 8 ? ph[0] : ph[1];
    const int64_t vph = grp < 2 ? ph[0] : ph[1];
    const uint16_t* kpage = kpool + (kph * Hkv + g) * (kPage * D);
    const uint16_t* vpage = vpool + (vph * Hkv + g) * (D * kPage);
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int c = 0; c < NQ; ++c)
        kf[v][c] = *reinterpret_cast<const bf16x8*>(kpage + (kslot0 + 4 * v) * D + c * 32 + grp * 8);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      vf[db] = *reinterpret_cast<const u32x4*>(vpage + (db * 16 + c16) * kPage + (grp & 1) * 8);
  };
  bf16x8 kf[2][NQ];
  u32x4 vf[NDB];
  load_pages(phys, kf, vf);
  // block-table entries of the next batch, requested one batch ahead so that
  // each batch's page loads issue without a table round trip before them
  int32_t nphys[kBatch];
  auto load_table_ahead = [&](int p_next) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) nphys[j] = table_at(min(p_next + 4 * j, p_end - 1));
  };
  load_table_ahead(p_first + 4 * kBatch);

  // rotate (pairs i, i + D/2) with rotation row csr and round to bf16: the
  // queries, and the new key with the query's rotation row
  auto rotate_round = [&](const u32x4* w_in, bool valid, const float (&csr)[NQ / 2][8][2], bf16x8* out) {
    float x[NQ][8];
#pragma unroll
    for (int c = 0; c < NQ; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = valid ? w_in[c][e] : 0u;
        x[c][2 * e] = __uint_as_float(w << 16);
        x[c][2 * e + 1] = __uint_as_float(w & 0xffff0000u);
      }
    if (a.rope) {
#pragma unroll
      for (int c = 0; c < NQ / 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float lo, hi;
          rotate_pair(x[c][e], x[c + NQ / 2][e], csr[c][e][0], csr[c][e][1], lo, hi);
          x[c][e] = lo;
          x[c + NQ / 2][e] = hi;
        }
    }
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[c][2 * e], x[c][2 * e + 1]);
      out[c] = __builtin_bit_cast(bf16x8, w);
    }
  };
  bf16x8 qf[NCH][NQ];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) rotate_round(qw[ch], hvalid[ch], cs[ch], qf[ch]);
  bf16x8 knew[NQ];
  if (owns_new) {
    rotate_round(kw, true, cs[0], knew);
    // write the new token to the cache: the wave whose page it is, key row by
    // the lanes of row r_new, value column by the lanes of its 4-slot group
    if (p_new >= p_begin && ((p_new - p_begin) & 3) == wave) {
      const int64_t ph = table_at(p_new);
      if (c16 == r_new) {
        uint16_t* kdst = kpool + ((ph * Hkv + g) * kPage + r_new) * D;
#pragma unroll
        for (int c = 0; c < NQ; ++c) *reinterpret_cast<bf16x8*>(kdst + c * 32 + grp * 8) = knew[c];
      }
      if (grp == (r_new >> 2)) {
        uint16_t* vdst = vpool + (ph * Hkv + g) * (D * kPage) + r_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db) vdst[(db * 16 + c16) * kPage] = static_cast<uint16_t>(vw[db]);
      }
    }
  }

  f32x4 o[NCH][NDB];
  float m_run[NCH], l_run[NCH];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[ch][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[ch] = -1e30f;
    l_run[ch] = 0.f;
  }

  // wave w takes pages p_begin + w, + 4, ...: a batch is p0 and p0 + 4 (a
  // second page past the split's end reloads its last page and is masked)
  for (int p0 = p_first; p0 < p_end; p0 += 4 * kBatch) {
    if (p0 != p_first) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j) phys[j] = nphys[j];
      load_pages(phys, kf, vf);
      load_table_ahead(p0 + 4 * kBatch);
    }
    const bool second = p0 + 4 < p_end;
    if (owns_new && (p_new == p0 || (second && p_new == p0 + 4))) {
      // slot T-1 from registers: whatever the page held there is ignored
      const int jn = p_new == p0 ? 0 : 1;
      if (c16 == 8 * jn + 4 * (r_new >> 3) + (r_new & 3)) {
        const int vn = (r_new >> 2) & 1;
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int c = 0; c < NQ; ++c)
            if (v == vn) kf[v][c] = knew[c];
      }
      if (grp == 2 * jn + (r_new >> 3)) {
        const int e = r_new & 7;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int w = 0; w < 4; ++w)
            if (w == (e >> 1)) {
              const uint32_t word = vf[db][w];
              vf[db][w] = (e & 1) ? ((word & 0x0000ffffu) | (vw[db] << 16)) : ((word & 0xffff0000u) | vw[db]);
            }
      }
    }
    // this lane's V^T slots: page p0 + 4*(grp/2), slots kv0 .. kv0 + 7; those
    // at or past the length, and all of a masked second page, are zeroed so
    // that 0 * NaN never occurs
    const bool dead = (grp >> 1) == 1 && !second;
    const int kv0 = (p0 + 4 * (grp >> 1)) * kPage + 8 * (grp & 1);
    if (dead || kv0 + 8 > T) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t keep = (!dead && kv0 + 2 * w < T ? 0x0000ffffu : 0u) |
                              (!dead && kv0 + 2 * w + 1 < T ? 0xffff0000u : 0u);
#pragma unroll
        for (int db = 0; db < NDB; ++db) vf[db][w] &= keep;
      }
    }
    const int p_last = second ? p0 + 4 : p0;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      if (ch > 0 && !two) break;
      // scores of keys kv0 + 4v + i (element i of half-block v) for this lane's column
      f32x4 s[2];
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        s[v] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NQ; ++c) s[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[v][c], qf[ch][c], s[v], 0, 0, 0);
      }
      if (dead) {
#pragma unroll
        for (int v = 0; v < 2; ++v) s[v] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
      if (p_last * kPage + kPage > start + 1) {
        // the block holds keys past the first query's position: causal mask
        // per column (covers the keys at or past T, since every qpos < T)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kv0 + 4 * v + i > qpos[ch]) s[v][i] = -INFINITY;
      }
      if (WIN && p0 * kPage < start + cnt - a.window) {
        // the block holds keys before the last column's window: per column
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kv0 + 4 * v + i <= qpos[ch] - a.window) s[v][i] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                       fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[ch], mx * sl2);
      const float alpha = __builtin_amdgcn_exp2f(m_run[ch] - m_new);
      m_run[ch] = m_new;
      float pr[8];
#pragma unroll
      for (int v = 0; v < 2; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[4 * v + i] = __builtin_amdgcn_exp2f(fmaf(s[v][i], sl2, -m_new));
      l_run[ch] = l_run[ch] * alpha + (((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7])));
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(pr[e]);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        o[ch][db] *= alpha;
        o[ch][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf[db]), pb, o[ch][db], 0, 0, 0);
      }
    }
  }

  // combine the four waves: lane (column c16, grp) holds o rows d = 16*db + 4*grp + i
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    float l_tot = l_run[ch] + __shfl_xor(l_run[ch], 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (grp == 0) {
      red_m[wave][ch * 16 + c16] = m_run[ch];
      red_l[wave][ch * 16 + c16] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) red_o[wave][ch * 16 + c16][db * 16 + grp * 4 + i] = o[ch][db][i];
  }
  __syncthreads();

  // 256 threads: column hh = tid / 16 of a chunk; thread dl holds d = E*dl .. E*dl + E-1
  constexpr int E = D / 16;
  const int hh = threadIdx.x >> 4;
  const int dl = threadIdx.x & 15;
  for (int ch = 0; ch < NCH; ++ch) {
    if (Gc[ch] <= 0) break;
    const int col = ch * 16 + hh;
    const bool hv2 = hh < Gc[ch];
    float M = red_m[0][col];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, red_m[w][col]);
    float L = 0.f;
    float acc[E];
    {
      float sc[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        sc[w] = __builtin_amdgcn_exp2f(red_m[w][col] - M);
        L += red_l[w][col] * sc[w];
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) v += red_o[w][col][E * dl + e] * sc[w];
        acc[e] = v;
      }
    }
    if (nsplit == 1) {
      if (hv2) {
        const float inv = 1.f / L;
        uint16_t* orow = out_row(ch, hh);
        uint32_t w[E / 2];
#pragma unroll
        for (int e = 0; e < E / 2; ++e) w[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
        if constexpr (E == 8)
          *reinterpret_cast<u32x4*>(orow + E * dl) = u32x4{w[0], w[1], w[2], w[3]};
        else
          *reinterpret_cast<u32x2*>(orow + E * dl) = u32x2{w[0], w[1]};
      }
      continue;
    }

    // Split records of this (sequence, kv head, column chunk): o rows
    // [split][column in chunk][D] and (m, l) headers [split][column in chunk],
    // written and read with device-scope (sc1) buffer accesses, which stay
    // coherent across the XCDs' L2 caches.  The last K splits are also
    // mergers: merger j combines output columns [j*D/K, (j+1)*D/K) of every
    // column.  Flags: one row of nsplit per merger, so a merger clears its own
    // row without racing another's wait.
    const int K = nsplit >= kDecodeMergers ? kDecodeMergers : 2;   // divides D/4
    const int mj = split - (nsplit - K);          // merger index, negative for the others
    const int yrow = g * hchunks + hcb0 + ch;
    const int64_t group = static_cast<int64_t>(a.split_off[b]) * gy + static_cast<int64_t>(yrow) * nsplit;
    int32_t* flags = a.flags + group * kDecodeMergers;
    const int gcc = Gc[ch];
    const __amdgpu_buffer_rsrc_t ro =
        __builtin_amdgcn_make_buffer_rsrc(a.part_o + group * (16 * D), 0, nsplit * gcc * D * 4, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rh =
        __builtin_amdgcn_make_buffer_rsrc(a.part_h + group * (16 * 2), 0, nsplit * gcc * 2 * 4, kBufferWord3);
    if (hv2) {
      const int rec = split * gcc + hh;
#pragma unroll
      for (int e = 0; e < E; e += 4)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]}), ro,
            (rec * D + E * dl + e) * 4, 0, kSc1);
      if (dl == 0)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, float2_t{M, L}), rh, rec * 8, 0, kSc1);
    }
    __builtin_amdgcn_s_waitcnt(0);        // this thread's record has reached the device
    __syncthreads();                      // (also: the previous chunk's merge no longer reads s_ok)
    if (static_cast<int>(threadIdx.x) < K && static_cast<int>(threadIdx.x) != mj)
      __hip_atomic_store(flags + threadIdx.x * nsplit + split, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (mj < 0) continue;

    // Merger: wait (bounded) for every other split's record.  Then each of this
    // merger's (column, d-run) pairs is spread over F adjacent lanes (F a power
    // of two), lane f taking splits f, f + F, ...: a few loads per thread, all
    // in flight together, a register-only combine with a running maximum, and
    // the F partials combined across lanes.
    int32_t* myflags = flags + mj * nsplit;
    if (threadIdx.x == 0) s_ok = 1;
    __syncthreads();
    for (int t = threadIdx.x; t < nsplit; t += 256) {
      if (t == split) continue;
      int spins = 0;
      while (__hip_atomic_load(myflags + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.wait_value) {
        if (spins >= a.spin_limit) {
          s_ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
        ++spins;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0 && !s_ok) __hip_atomic_store(a.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int CK = (D / 4) / K;              // float4 runs of a column owned by this merger
    const int P = gcc * CK;                  // (column, run) pairs, at most 256
    int F = 1;                               // lanes per pair: largest power of two with P*F <= 256, at most 16
    while (F < 16 && P * F * 2 <= 256) F *= 2;
    const int t = threadIdx.x;
    const int pr = t / F;
    const int f = t & (F - 1);
    const bool pv = pr < P;
    const int ph = pv ? pr / CK : 0;
    const int pc = mj * CK + pr % CK;
    float Mr = -INFINITY;
    float Lr = 0.f;
    f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
    if (pv) {
      for (int s0 = f; s0 < nsplit; s0 += F * kMergeBatch) {
        float2_t hm[kMergeBatch];
        f32x4 v[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
          const int rec = min(s0 + u * F, nsplit - 1) * gcc + ph;
          hm[u] = __builtin_bit_cast(float2_t, __builtin_amdgcn_raw_buffer_load_b64(rh, rec * 8, 0, kSc1));
          v[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, (rec * D + 4 * pc) * 4, 0, kSc1));
        }
        // s0 < nsplit, so hm[0] is valid and mx is finite
        float mx = Mr;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) mx = fmaxf(mx, s0 + u * F < nsplit ? hm[u].x : -INFINITY);
        const float sc = __builtin_amdgcn_exp2f(Mr - mx);
        acc4 *= sc;
        Lr *= sc;
        Mr = mx;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
          const float e = __builtin_amdgcn_exp2f(hm[u].x - mx);
          const float w = s0 + u * F < nsplit ? e : 0.f;
          acc4 += v[u] * w;
          Lr += hm[u].y * w;
        }
      }
    }
    // combine the F lanes of each pair (a lane that took no split holds m = -inf, l = 0)
    float Mg = Mr;
    for (int x = 1; x < F; x <<= 1) Mg = fmaxf(Mg, __shfl_xor(Mg, x));
    const float w = Mr == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mr - Mg);
    float Lg = Lr * w;
    f32x4 o4 = acc4 * w;
    for (int x = 1; x < F; x <<= 1) {
      Lg += __shfl_xor(Lg, x);
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] += __shfl_xor(o4[e], x);
    }
    if (pv && f == 0) {
      const float inv = s_ok ? 1.f / Lg : __builtin_nanf("");
      uint16_t* orow = out_row(ch, ph);
      *reinterpret_cast<u32x2*>(orow + 4 * pc) =
          u32x2{pack_bf16x2(o4[0] * inv, o4[1] * inv), pack_bf16x2(o4[2] * inv, o4[3] * inv)};
    }
    // leave this merger's flag row at zero for the next call
    for (int t2 = threadIdx.x; t2 < nsplit; t2 += 256)
      if (t2 != split) __hip_atomic_store(myflags + t2, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

hipError_t launch_decode_bf16(const DecodeArgs& a, int total_splits, hipStream_t s) {
  const int hchunks = (a.ncol + 15) / 16;
  bool chunk = a.ncol != a.Hq / a.Hkv || a.n_rect != 1;
  for (int j = 0; j < a.nseq && !chunk; ++j) chunk = a.meta.count[j] != 1 || a.meta.row0[j] != 0;
  // chunk mode: two column chunks per workgroup
  const dim3 grid = chunk ? dim3(total_splits * ((hchunks + 1) / 2) * a.Hkv) : dim3(total_splits, a.Hkv * hchunks);
  const bool win = a.window != 0;
  bool newp = false;
  for (int j = 0; j < a.nseq && !chunk; ++j) newp = newp || a.new_page[j] >= 0;
  auto pick = [&](auto dv, auto cv, auto wv) {
    if (newp)
      hipLaunchKernelGGL((decode_bf16_kernel<decltype(dv)::value, decltype(cv)::value, decltype(wv)::value, true>),
                         grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_bf16_kernel<decltype(dv)::value, decltype(cv)::value, decltype(wv)::value, false>),
                         grid, dim3(256), 0, s, a);
  };
  using D128 = std::integral_constant<int, 128>;
  using D64 = std::integral_constant<int, 64>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (a.d == 128) {
    if (chunk) win ? pick(D128(), T_(), T_()) : pick(D128(), T_(), F_());
    else win ? pick(D128(), F_(), T_()) : pick(D128(), F_(), F_());
  } else {
    if (chunk) win ? pick(D64(), T_(), T_()) : pick(D64(), T_(), F_());
    else win ? pick(D64(), F_(), T_()) : pick(D64(), F_(), F_());
  }
  return hipGetLastError();
}

}  // namespace gqa
