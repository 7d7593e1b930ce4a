// Kernel-argument structs shared by the host entry points and the kernels.
// Every per-call piece of metadata travels in the kernel-argument segment, so a
// launch never waits on a host-to-device copy.
#pragma once
#include <cstdint>
#include <hip/hip_runtime.h>

namespace gqa {

constexpr int kPage = 16;          // tokens per page
constexpr int kMaxSeqPerLaunch = 64;
constexpr int kMaxRunsPerLaunch = 144;   // entries of one attention launch
constexpr int kMaxRowsPerLaunch = 64;    // batch rows of one attention launch (row index fits 8 bits)
constexpr int kMaxCopiesPerLaunch = 496;  // page copies per launch; the arguments stay under 4 KiB
constexpr int kMaxPatchPerLaunch = 672;   // block-table entries per launch (16-bit offsets from a base
                                          // index, 32-bit pages: the arguments stay under 4 KiB)
constexpr int kMaxSplitDecode = 128;   // splits per sequence in one decode launch
constexpr int kDecodeMergers = 4;      // splits of a sequence that combine the split records
constexpr int64_t kStaticScratchBytes = int64_t{48} << 20;   // the library's static split-T scratch per device

// Per-entry metadata of one launch (an entry is one run of valid tokens of a
// sequence, or a whole decode row).
//  start: position of the entry's first token (the cache length before an
//         append plus the valid tokens of earlier runs of the row; T-1 for a
//         decode query);
//  count: tokens (queries) of the entry;
//  row0:  rectangular row of its first token;
//  total: cache length the attention reads (keys at slots >= total are never
//         valid, whatever the page holds).
//  brow:  batch row of Q/K/V/O the entry reads and writes (a row whose valid
//         tokens have holes gives one entry per run of consecutive valid rows);
//  zlo, zhi: rectangular rows [zlo, zhi) whose padding (rows outside
//         [row0, row0 + count)) the entry writes as 0.
struct SeqMeta {
  int32_t seq[kMaxSeqPerLaunch];
  int32_t brow[kMaxSeqPerLaunch];
  int32_t start[kMaxSeqPerLaunch];
  int32_t count[kMaxSeqPerLaunch];
  int32_t row0[kMaxSeqPerLaunch];
  int32_t total[kMaxSeqPerLaunch];
  int32_t zlo[kMaxSeqPerLaunch];
  int32_t zhi[kMaxSeqPerLaunch];
};

// Entries of one attention launch, kept compact so that a row whose valid
// tokens have many holes still fits few launches: per entry (a run of valid
// rows) its first position, token count, first rectangular row, padding share
// [zlo, zhi) and the index of its batch row in the per-row arrays; per batch
// row its sequence, the batch row itself and the cache length read.
struct AttnMeta {
  int32_t start[kMaxRunsPerLaunch];
  int32_t count[kMaxRunsPerLaunch];
  int32_t row0[kMaxRunsPerLaunch];
  int32_t zlo[kMaxRunsPerLaunch];
  int32_t zhi[kMaxRunsPerLaunch];
  uint8_t row[kMaxRunsPerLaunch];
  int32_t seq[kMaxRowsPerLaunch];
  int32_t brow[kMaxRowsPerLaunch];
  int32_t total[kMaxRowsPerLaunch];
};

struct PatchArgs {
  int32_t* table;
  int32_t n;
  int32_t base;                         // entry i goes to table[base + offset[i]]
  uint16_t offset[kMaxPatchPerLaunch];
  int32_t value[kMaxPatchPerLaunch];
};

struct AppendArgs {
  const void* K;
  const void* V;
  int64_t k_s0, k_s1, k_s2;   // element strides: batch, head, token
  int64_t v_s0, v_s1, v_s2;
  void* k_pool;               // this layer's pool base
  void* v_pool;
  const int32_t* table;
  int32_t table_w;
  int32_t window;             // sliding window (0: none); a windowed cache is a ring of table_w pages
  int32_t Hkv, d, nseq;
  const float* rope;          // [max_position][d/2][2] or nullptr
  SeqMeta meta;
};

struct AttnArgs {
  const void* Q;
  int64_t q_s0, q_s1, q_s2;
  void* O;
  int64_t o_s0, o_s1, o_s2;
  const void* k_pool;
  const void* v_pool;
  const int32_t* table;
  int32_t table_w;
  int32_t window;             // sliding window (0: none); a windowed cache is a ring of table_w pages
  int32_t Hq, Hkv, d, n_rect, nseq;
  float scale;                // 1/sqrt(d)
  float scale_log2;           // log2(e)/sqrt(d)
  uint32_t pool_bytes;        // bytes of this layer's K (= V) pool; offsets into it fit 32 bits
  const float* rope;          // [max_position][d/2][2] or nullptr
  const float* rope_t;        // the same values by 16-byte chunk: [d/8][max_position][4] floats
  int32_t rope_rows;          // max_position
  AttnMeta meta;              // nseq entries
};

struct DecodeArgs {
  const void* q;
  int64_t q_s0, q_s1, q_s2;   // element strides: batch, head, token
  void* o;
  int64_t o_s0, o_s1, o_s2;
  const void* k_new;          // optional new token appended by the same launch: [B][Hkv][1][d]
  int64_t kn_s0, kn_s1;
  const void* v_new;
  int64_t vn_s0, vn_s1;
  void* k_pool;               // this layer's pool base (written only for the new token)
  void* v_pool;
  int32_t* table;             // read; written only for new_page entries
  int32_t table_w;
  int32_t window;             // sliding window (0: none); a windowed cache is a ring of table_w pages
  int32_t Hq, Hkv, d, nseq;
  int32_t ncol;               // (token, head) columns per kv head: tokens of the longest chunk x Hq/Hkv
  int32_t n_rect;             // rows of the rectangular q / o (padding rows of o are zeroed)
  int32_t pages_per_split;
  float scale_log2;
  const float* rope;
  float* part_o;              // split o rows [split][y][16][d]
  float* part_h;              // split (m, l) headers [split][y][16][2]
  int32_t* flags;             // ready flags [split group][merger][split]; zero between calls
  int32_t* status;            // sticky failure word of the workspace (set when a merge gives up)
  int32_t epoch;              // nonzero value a split writes into its ready flags for this call
  int32_t wait_value;         // flag value the mergers wait for (epoch, unless a test forces a give-up)
  int32_t spin_limit;         // polls of one ready flag before a merger gives up
  int32_t split_off[kMaxSeqPerLaunch + 1];
  // physical page of the new token's slot when this call opens that page (-1
  // otherwise): the launch takes it from here and writes its block-table
  // entry, instead of a separate block-table patch launch before it
  int32_t new_page[kMaxSeqPerLaunch];
  SeqMeta meta;               // start: position of the first query token; count: query tokens;
                              // row0: their first rectangular row; total: keys read (start + count)
};


struct CopyArgs {
  void* k_pool;               // whole pool (all layers)
  void* v_pool;
  int64_t layer_stride;       // elements per layer of a pool
  int64_t page_elems;         // elements of one page (all kv heads)
  int32_t n;
  int32_t elt_bytes;
  int32_t src[kMaxCopiesPerLaunch];
  int32_t dst[kMaxCopiesPerLaunch];
};

// Every argument block stays within 4 KiB, the kernel-argument size every
// launch path takes.
static_assert(sizeof(AttnArgs) <= 4096, "attention arguments exceed 4 KiB");
static_assert(sizeof(DecodeArgs) <= 4096, "decode arguments exceed 4 KiB");
static_assert(sizeof(AppendArgs) <= 4096, "append arguments exceed 4 KiB");
static_assert(sizeof(PatchArgs) <= 4096, "block-table patch arguments exceed 4 KiB");
static_assert(sizeof(CopyArgs) <= 4096, "page copy arguments exceed 4 KiB");

hipError_t launch_table_patch(const PatchArgs& a, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, int dtype, int grid_x, hipStream_t s);
hipError_t launch_attend_f32(const AttnArgs& a, hipStream_t s);
hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, int total_splits, hipStream_t s);
hipError_t launch_page_copy(const CopyArgs& a, int num_layers, hipStream_t s);
// Device address of the static split-T scratch on the current device; the
// first call on a device resolves it and zero-fills its first zero_bytes on s.
hipError_t static_scratch(int64_t zero_bytes, hipStream_t s, void** out);

}  // namespace gqa
