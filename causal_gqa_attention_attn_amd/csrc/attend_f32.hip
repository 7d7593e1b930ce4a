// Generic float32 attention over the paged cache, one thread per query row.
//
// Definition (page "Prefill：整层状态演化与 KV 建立", sections 2.2-2.3): query
// head h reads KV head g(h) = floor(h*Hkv/Hq); a valid query at position p
// reads the cache slots j <= p; S = <rot(q), k_used>/sqrt(d); the softmax is
// row-stable over the finite scores; O = sum_j A_j v_j.  Padding rows get 0.
// Used for float32 caches of any head dimension <= 128 (prefill and decode);
// the running maximum and sum are updated one key at a time.
#include "common.hpp"
#include "device.hpp"

namespace gqa {

// grid: x = block of 64 rectangular rows, y = query head, z = sequence
template <int DMAX>
__global__ __launch_bounds__(64) void attend_f32_kernel(AttnArgs a) {
  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int r = blockIdx.x * 64 + threadIdx.x;
  if (r >= a.n_rect) return;
  const int d = a.d;
  const int seq = a.meta.seq[a.meta.row[b]];
  const int c0 = a.meta.start[b];
  const int nb = a.meta.count[b];
  const int r0 = a.meta.row0[b];
  const int br = a.meta.brow[a.meta.row[b]];
  float* orow = static_cast<float*>(a.O) + br * a.o_s0 + h * a.o_s1 + static_cast<int64_t>(r) * a.o_s2;
  if (r < r0 || r >= r0 + nb) {
    if (r >= a.meta.zlo[b] && r < a.meta.zhi[b])
      for (int e = 0; e < d; ++e) orow[e] = 0.f;
    return;
  }
  const int pos = c0 + (r - r0);
  const int g = h / (a.Hq / a.Hkv);
  const float* qrow = static_cast<const float*>(a.Q) + br * a.q_s0 + h * a.q_s1 + static_cast<int64_t>(r) * a.q_s2;
  // rotated query, read pairwise from memory: q'[i] = x c - y s, q'[i+d/2] = x s + y c
  float q[DMAX];
  const int half = d / 2;
#pragma unroll
  for (int e = 0; e < DMAX; ++e) {
    q[e] = 0.f;
    if (e < d) {
      if (a.rope) {
        const bool lo = e < half;
        const int i = lo ? e : e - half;
        const float c = a.rope[(static_cast<int64_t>(pos) * half + i) * 2];
        const float s = a.rope[(static_cast<int64_t>(pos) * half + i) * 2 + 1];
        float xo, yo;
        rotate_pair(qrow[i], qrow[i + half], c, s, xo, yo);
        q[e] = lo ? xo : yo;
      } else {
        q[e] = qrow[e];
      }
    }
  }
  const float* kpool = static_cast<const float*>(a.k_pool);
  const float* vpool = static_cast<const float*>(a.v_pool);
  const int32_t* trow = a.table + static_cast<int64_t>(seq) * a.table_w;
  float acc[DMAX];
#pragma unroll
  for (int e = 0; e < DMAX; ++e) acc[e] = 0.f;
  float m = -INFINITY;
  float l = 0.f;
  for (int j = a.window ? max(0, pos - a.window + 1) : 0; j <= pos; ++j) {
    const int64_t phys = trow[a.window ? (j / kPage) % a.table_w : j / kPage];
    const float* krow = kpool + ((phys * a.Hkv + g) * kPage + (j % kPage)) * d;
    const float* vcol = vpool + (phys * a.Hkv + g) * d * kPage + (j % kPage);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < DMAX; ++e)
      if (e < d) s += q[e] * krow[e];
    s *= a.scale;
    if (s > m) {
      const float alpha = expf(m - s);
      l = l * alpha + 1.f;
#pragma unroll
      for (int e = 0; e < DMAX; ++e)
        if (e < d) acc[e] = acc[e] * alpha + vcol[e * kPage];
      m = s;
    } else {
      const float p = expf(s - m);
      l += p;
#pragma unroll
      for (int e = 0; e < DMAX; ++e)
        if (e < d) acc[e] += p * vcol[e * kPage];
    }
  }
  const float inv = 1.f / l;
  for (int e = 0; e < d; ++e) orow[e] = acc[e] * inv;
}

hipError_t launch_attend_f32(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.n_rect + 63) / 64, a.Hq, a.nseq);
  if (a.d <= 8)
    hipLaunchKernelGGL(attend_f32_kernel<8>, grid, dim3(64), 0, s, a);
  else if (a.d <= 32)
    hipLaunchKernelGGL(attend_f32_kernel<32>, grid, dim3(64), 0, s, a);
  else if (a.d <= 64)
    hipLaunchKernelGGL(attend_f32_kernel<64>, grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(attend_f32_kernel<128>, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace gqa
