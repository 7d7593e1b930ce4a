// Cache-side kernels: block-table patches, the fused rotation + paged cache
// write, and physical page copies.
//
// Cache contract (page "Prefill：整层状态演化与 KV 建立", section 2.5): the
// cache holds the keys actually used by attention, i.e. after the position
// rotation, plus the values, at slot = position.  Paging (page "KV Cache 与
// Prefill/Decode 推理路径", PagedAttention lesson): slot t lives in logical page
// t / 16 at offset t % 16; the block table maps logical to physical pages.
//
// Physical layout per layer:  K  [page][kv head][16 slots][d]
//                             V  [page][kv head][d][16 slots]   (V^T per page)
// so attention kernels read a K page row-major and a V page already transposed,
// which is the operand order the matrix cores want for S = K q and O^T = V^T P^T.
#include "common.hpp"
#include "device.hpp"

namespace gqa {

__global__ __launch_bounds__(256) void table_patch_kernel(PatchArgs a) {
  for (int i = threadIdx.x; i < a.n; i += blockDim.x) a.table[a.base + a.offset[i]] = a.value[i];
}

hipError_t launch_table_patch(const PatchArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(table_patch_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16(x); }

// grid: x = logical page within the call's slot range, y = kv head, z = sequence.
// Each block writes the slots of one (page, head) that this call appends.
template <typename T>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int nb = a.meta.count[b];
  if (nb == 0) return;
  const int seq = a.meta.seq[b];
  const int c0 = a.meta.start[b];
  const int r0 = a.meta.row0[b];
  const int lp = c0 / kPage + static_cast<int>(blockIdx.x);
  const int slot_lo = max(c0, lp * kPage);
  const int slot_hi = min(c0 + nb, lp * kPage + kPage);
  if (slot_lo >= slot_hi) return;
  const int nslots = slot_hi - slot_lo;
  const int d = a.d;
  const int half = d / 2;
  const int64_t phys = a.table[static_cast<int64_t>(seq) * a.table_w + (a.window ? lp % a.table_w : lp)];
  T* kp = static_cast<T*>(a.k_pool) + (phys * a.Hkv + g) * (kPage * d);
  T* vp = static_cast<T*>(a.v_pool) + (phys * a.Hkv + g) * (d * kPage);
  const T* kin = static_cast<const T*>(a.K) + a.meta.brow[b] * a.k_s0 + g * a.k_s1;
  const T* vin = static_cast<const T*>(a.V) + a.meta.brow[b] * a.v_s0 + g * a.v_s1;

  // keys: rotate in float32 (pairs i, i + d/2), round to the storage dtype
  for (int e = threadIdx.x; e < nslots * d; e += blockDim.x) {
    const int si = e / d;
    const int dd = e - si * d;
    const int slot = slot_lo + si;
    const T* row = kin + static_cast<int64_t>(r0 + slot - c0) * a.k_s2;
    T out;
    if (a.rope) {
      const bool lo = dd < half;
      const int i = lo ? dd : dd - half;
      const float c = a.rope[(static_cast<int64_t>(slot) * half + i) * 2];
      const float s = a.rope[(static_cast<int64_t>(slot) * half + i) * 2 + 1];
      const float own = to_f32<T>(row[dd]);
      const float other = to_f32<T>(row[lo ? dd + half : dd - half]);
      float xo, yo;
      if (lo) {
        rotate_pair(own, other, c, s, xo, yo);
        out = from_f32<T>(xo);
      } else {
        rotate_pair(other, own, c, s, xo, yo);
        out = from_f32<T>(yo);
      }
    } else {
      out = row[dd];
    }
    kp[(slot % kPage) * d + dd] = out;
  }
  // values: bit copy into the d-major page
  for (int e = threadIdx.x; e < nslots * d; e += blockDim.x) {
    const int dd = e / nslots;
    const int si = e - dd * nslots;
    const int slot = slot_lo + si;
    vp[dd * kPage + (slot % kPage)] = vin[static_cast<int64_t>(r0 + slot - c0) * a.v_s2 + dd];
  }
}

// bfloat16 caches: the same writes in 16-byte units.  grid as above.
//  * keys: a thread takes 8 dims of a slot and the 8 dims they pair with
//    (i and i + D/2), rotates them in float32 exactly as the scalar path does
//    and writes both 16-byte runs;
//  * values: the page's rows are staged in LDS, then each thread writes 8
//    consecutive slots of one d-row of the d-major page; a run that the call
//    only partly covers keeps the slots it does not cover.
template <int D>
__global__ __launch_bounds__(256) void append_bf16_kernel(AppendArgs a) {
  constexpr int PAIRS = D / 16;                 // 8-dim runs per half row
  __shared__ __attribute__((aligned(16))) uint16_t vt[kPage][D + 8];
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int nb = a.meta.count[b];
  if (nb == 0) return;
  const int seq = a.meta.seq[b];
  const int c0 = a.meta.start[b];
  const int lp = c0 / kPage + static_cast<int>(blockIdx.x);
  const int slot_lo = max(c0, lp * kPage);
  if (slot_lo >= min(c0 + nb, lp * kPage + kPage)) return;
  // Runs of one row (padding between its valid tokens) can share a page: the
  // 16-byte value writes below merge slots, so one workgroup, that of the
  // first run on the page, writes the page's slots of every run of the row.
  const int brow = a.meta.brow[b];
  if (b > 0 && a.meta.brow[b - 1] == brow && (a.meta.start[b - 1] + a.meta.count[b - 1] - 1) / kPage == lp) return;
  int last = b;
  while (last + 1 < a.nseq && a.meta.brow[last + 1] == brow && a.meta.start[last + 1] < lp * kPage + kPage) ++last;
  const int slot_hi = min(a.meta.start[last] + a.meta.count[last], lp * kPage + kPage);
  // rectangular row of a slot of this page
  auto src_row = [&](int slot) {
    int j = b;
    while (j < last && slot >= a.meta.start[j] + a.meta.count[j]) ++j;
    return a.meta.row0[j] + slot - a.meta.start[j];
  };
  const int64_t phys = a.table[static_cast<int64_t>(seq) * a.table_w + (a.window ? lp % a.table_w : lp)];
  uint16_t* kp = static_cast<uint16_t*>(a.k_pool) + (phys * a.Hkv + g) * (kPage * D);
  uint16_t* vp = static_cast<uint16_t*>(a.v_pool) + (phys * a.Hkv + g) * (D * kPage);
  const uint16_t* kin = static_cast<const uint16_t*>(a.K) + a.meta.brow[b] * a.k_s0 + g * a.k_s1;
  const uint16_t* vin = static_cast<const uint16_t*>(a.V) + a.meta.brow[b] * a.v_s0 + g * a.v_s1;
  const int t = threadIdx.x;

  // keys
  if (t < kPage * PAIRS) {
    const int si = t / PAIRS;
    const int p = t - si * PAIRS;
    const int slot = lp * kPage + si;
    if (slot >= slot_lo && slot < slot_hi) {
      const uint16_t* row = kin + static_cast<int64_t>(src_row(slot)) * a.k_s2;
      const u32x4 wlo = *reinterpret_cast<const u32x4*>(row + 8 * p);
      const u32x4 whi = *reinterpret_cast<const u32x4*>(row + D / 2 + 8 * p);
      u32x4 olo = wlo, ohi = whi;
      if (a.rope) {
        const float* rr = a.rope + (static_cast<int64_t>(slot) * (D / 2) + 8 * p) * 2;
        f32x4 cs[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) cs[q] = *reinterpret_cast<const f32x4*>(rr + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x[2], y[2], xo[2], yo[2];
          x[0] = __uint_as_float(wlo[e] << 16);
          x[1] = __uint_as_float(wlo[e] & 0xffff0000u);
          y[0] = __uint_as_float(whi[e] << 16);
          y[1] = __uint_as_float(whi[e] & 0xffff0000u);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int i = 2 * e + h;            // pair 8p + i: (cos, sin) at rr[2i], rr[2i + 1]
            const float c = cs[i / 2][(i % 2) * 2];
            const float sn = cs[i / 2][(i % 2) * 2 + 1];
            rotate_pair(x[h], y[h], c, sn, xo[h], yo[h]);
          }
          olo[e] = pack_bf16x2(xo[0], xo[1]);
          ohi[e] = pack_bf16x2(yo[0], yo[1]);
        }
      }
      uint16_t* krow = kp + (slot % kPage) * D;
      *reinterpret_cast<u32x4*>(krow + 8 * p) = olo;
      *reinterpret_cast<u32x4*>(krow + D / 2 + 8 * p) = ohi;
    }
  }
  // values: rows of the page into LDS (slots the call does not write stay unread)
  for (int e = t; e < kPage * (D / 8); e += 256) {
    const int si = e / (D / 8);
    const int ch = e - si * (D / 8);
    const int slot = lp * kPage + si;
    if (slot >= slot_lo && slot < slot_hi)
      *reinterpret_cast<u32x4*>(&vt[si][ch * 8]) =
          *reinterpret_cast<const u32x4*>(vin + static_cast<int64_t>(src_row(slot)) * a.v_s2 + ch * 8);
  }
  __syncthreads();
  for (int e = t; e < D * 2; e += 256) {
    const int dr = e >> 1;
    const int h8 = e & 1;
    const int s0 = lp * kPage + h8 * 8;
    if (s0 + 8 <= slot_lo || s0 >= slot_hi) continue;
    uint16_t* dst = vp + dr * kPage + h8 * 8;
    u32x4 w;
    const bool whole = s0 >= slot_lo && s0 + 8 <= slot_hi;
    if (!whole) w = *reinterpret_cast<const u32x4*>(dst);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t lo = w[q] & 0xffffu, hi = w[q] >> 16;
      const int sa = s0 + 2 * q, sb = sa + 1;
      if (whole || (sa >= slot_lo && sa < slot_hi)) lo = vt[h8 * 8 + 2 * q][dr];
      if (whole || (sb >= slot_lo && sb < slot_hi)) hi = vt[h8 * 8 + 2 * q + 1][dr];
      w[q] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(dst) = w;
  }
}

hipError_t launch_append(const AppendArgs& a, int dtype, int grid_x, hipStream_t s) {
  dim3 grid(grid_x, a.Hkv, a.nseq);
  if (dtype == 0)
    hipLaunchKernelGGL(append_kernel<float>, grid, dim3(256), 0, s, a);
  else if (a.d == 128)
    hipLaunchKernelGGL(append_bf16_kernel<128>, grid, dim3(256), 0, s, a);
  else if (a.d == 64)
    hipLaunchKernelGGL(append_bf16_kernel<64>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// grid: x = pair, y = layer, z = 0 for K, 1 for V.  Copies one page of all kv
// heads in 16-byte units.
__global__ __launch_bounds__(256) void page_copy_kernel(CopyArgs a) {
  const int i = blockIdx.x;
  const int64_t layer = blockIdx.y;
  char* pool = static_cast<char*>(blockIdx.z == 0 ? a.k_pool : a.v_pool);
  const int64_t page_bytes = a.page_elems * a.elt_bytes;
  const int64_t layer_bytes = a.layer_stride * a.elt_bytes;
  const u32x4* src = reinterpret_cast<const u32x4*>(pool + layer * layer_bytes + a.src[i] * page_bytes);
  u32x4* dst = reinterpret_cast<u32x4*>(pool + layer * layer_bytes + a.dst[i] * page_bytes);
  const int64_t n16 = page_bytes / 16;
  for (int64_t e = threadIdx.x; e < n16; e += blockDim.x) dst[e] = src[e];
}

hipError_t launch_page_copy(const CopyArgs& a, int num_layers, hipStream_t s) {
  hipLaunchKernelGGL(page_copy_kernel, dim3(a.n, num_layers, 2), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gqa
