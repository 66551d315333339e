// Kernels around the flash loop: the KV-cache write, the cos/sin table and
// the split-KV combine.
#include "common.h"

namespace minipic {

// ---------------------------------------------------------------------------
// KV-cache write ("MiniPIC: Flexible Position-Independent Caching in <100LOC",
// abstract and §3.2: the cache holds unrotated K; V unchanged). One
// work-group stores 16 consecutive new tokens of one KV head. K rows are
// copied in 16-byte pieces. V is stored transposed per block ([d][16]); when
// the 16 tokens fill one block in order (the usual case for a freshly
// computed span) the transpose goes through LDS and every store is a full
// 16-byte row piece, otherwise each element is stored on its own.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) write_kv_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                       const int64_t* __restrict__ slots, int64_t n,
                                                       int hkv, T* __restrict__ kc, T* __restrict__ vc,
                                                       int64_t num_blocks) {
  constexpr int E = 16 / sizeof(T);     // elements per 16-byte piece
  constexpr int PIECES = kBlock * D / E;
  __shared__ __attribute__((aligned(16))) T tile[kBlock][D + E];
  __shared__ int64_t sl[kBlock];
  __shared__ int fast;
  const int g = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kBlock;
  const int tid = threadIdx.x;
  const int64_t cap = num_blocks * kBlock;
  if (tid < kBlock) {
    const int64_t tk = t0 + tid;
    int64_t s = tk < n ? slots[tk] : -1;
    if (s >= cap) s = -1;
    sl[tid] = s;
  }
  __syncthreads();
  if (tid == 0) {
    int f = sl[0] >= 0 && (sl[0] % kBlock) == 0;
    for (int i = 1; i < kBlock && f; ++i) f = sl[i] == sl[0] + i;
    fast = f;
  }
  for (int u = tid; u < PIECES; u += 256) {
    const int tok = u / (D / E);
    const int piece = u % (D / E);
    const int64_t s = sl[tok];
    if (s < 0) continue;
    const int64_t src = ((t0 + tok) * hkv + g) * D + piece * E;
    const u32x4 kv = *(const u32x4*)(k + src);
    *(u32x4*)(kc + (((s / kBlock) * hkv + g) * kBlock + s % kBlock) * D + piece * E) = kv;
    const u32x4 vv = *(const u32x4*)(v + src);
    *(u32x4*)(&tile[tok][piece * E]) = vv;
  }
  __syncthreads();
  if (fast) {
    const int64_t blk = sl[0] / kBlock;
    // V^T rows: D rows of 16 keys = 16/E pieces each
    for (int u = tid; u < D * (kBlock / E); u += 256) {
      const int d = u / (kBlock / E);
      const int kp = u % (kBlock / E);
      T buf[E];
#pragma unroll
      for (int j = 0; j < E; ++j) buf[j] = tile[kp * E + j][d];
      u32x4 pk;
      __builtin_memcpy(&pk, buf, 16);
      *(u32x4*)(vc + ((blk * hkv + g) * D + d) * kBlock + kp * E) = pk;
    }
  } else {
    for (int u = tid; u < kBlock * D; u += 256) {
      const int tok = u / D;
      const int d = u % D;
      const int64_t s = sl[tok];
      if (s < 0) continue;
      vc[(((s / kBlock) * hkv + g) * D + d) * kBlock + s % kBlock] = tile[tok][d];
    }
  }
}

hipError_t launch_write_kv(const void* k, const void* v, const int64_t* slots, int64_t n, int hkv, int D,
                           void* kc, void* vc, int64_t num_blocks, int dtype, hipStream_t s) {
  const dim3 grid((unsigned)((n + kBlock - 1) / kBlock), (unsigned)hkv);
  if (dtype == MINIPIC_BF16) {
    if (D == 128)
      hipLaunchKernelGGL((write_kv_kernel<uint16_t, 128>), grid, dim3(256), 0, s, (const uint16_t*)k,
                         (const uint16_t*)v, slots, n, hkv, (uint16_t*)kc, (uint16_t*)vc, num_blocks);
    else
      hipLaunchKernelGGL((write_kv_kernel<uint16_t, 64>), grid, dim3(256), 0, s, (const uint16_t*)k,
                         (const uint16_t*)v, slots, n, hkv, (uint16_t*)kc, (uint16_t*)vc, num_blocks);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((write_kv_kernel<uint32_t, 128>), grid, dim3(256), 0, s, (const uint32_t*)k,
                         (const uint32_t*)v, slots, n, hkv, (uint32_t*)kc, (uint32_t*)vc, num_blocks);
    else
      hipLaunchKernelGGL((write_kv_kernel<uint32_t, 64>), grid, dim3(256), 0, s, (const uint32_t*)k,
                         (const uint32_t*)v, slots, n, hkv, (uint32_t*)kc, (uint32_t*)vc, num_blocks);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// cos/sin table for the rotate-half RoPE of the in-kernel lookup
// ("MiniPIC ...", §3.2.2): row p = [cos(p theta_i) | sin(p theta_i)],
// theta_i = base^(-2i/d), angles and sin/cos in float64, rounded once.
// ---------------------------------------------------------------------------
__global__ void rope_table_kernel(float* cs, int max_pos, int d, double base) {
  const int half = d / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)max_pos * half) return;
  const int p = (int)(idx / half);
  const int i = (int)(idx % half);
  const double theta = pow(base, -2.0 * (double)i / (double)d);
  const double ang = (double)p * theta;
  double s, c;
  sincos(ang, &s, &c);
  cs[(int64_t)p * d + i] = (float)c;
  cs[(int64_t)p * d + half + i] = (float)s;
}

hipError_t launch_rope_table(float* cs, int max_pos, int d, double base, hipStream_t s) {
  const int64_t n = (int64_t)max_pos * (d / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, cs, max_pos, d,
                     base);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-KV combine: merge the partial (O, m, l) of the key splits of every
// q tile that was split, with weights 2^(m_s - max_s m_s) (log2 units).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) combine_kernel(AttnParams P, int bq, int G) {
  const int64_t bid = blockIdx.x;
  const int g = (int)(bid % P.hkv);
  const int64_t rest = bid / P.hkv;
  const int qt = (int)(rest % P.num_q_tiles);
  const int r = (int)(rest / P.num_q_tiles);
  const int qb = P.q_indptr[r], qe = P.q_indptr[r + 1];
  const int row0 = qb + qt * bq;
  if (row0 >= qe) return;
  const int ns = P.tile_nsplit[((int64_t)r * P.num_q_tiles + qt) * P.hkv + g];
  if (ns <= 1) return;
  const int nq = min(bq, qe - row0);
  const int units = nq * G * (D / 4);
  for (int u = threadIdx.x; u < units; u += 256) {
    const int d4 = u % (D / 4);
    const int rg = u / (D / 4);
    const int tok = rg / G;
    const int head = g * G + rg % G;
    const int64_t qrow = row0 + tok;
    float mstar = -INFINITY;
    for (int s = 0; s < ns; ++s) mstar = fmaxf(mstar, P.part_ml[((int64_t)s * P.total_q + qrow) * P.hq + head].x);
    float den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < ns; ++s) {
      const int64_t pr = ((int64_t)s * P.total_q + qrow) * P.hq + head;
      const float2 ml = P.part_ml[pr];
      if (ml.x == -INFINITY) continue;
      const float wgt = exp2f(ml.x - mstar);
      den += wgt * ml.y;
      const f32x4 po = *(const f32x4*)(P.part_o + pr * D + 4 * d4);
      num += wgt * po;
    }
    const float inv = 1.f / den;
    T* op = (T*)P.out + (qrow * P.hq + head) * D + 4 * d4;
    if constexpr (sizeof(T) == 4) {
      *(f32x4*)op = num * inv;
    } else {
      u32x2 pk;
      pk[0] = pack_bf16x2(num[0] * inv, num[1] * inv);
      pk[1] = pack_bf16x2(num[2] * inv, num[3] * inv);
      *(u32x2*)op = pk;
    }
  }
}

hipError_t launch_combine(const AttnParams& p, int D, int dtype, int bq, int G, int64_t grid, hipStream_t s) {
  if (dtype == MINIPIC_BF16) {
    if (D == 128) hipLaunchKernelGGL((combine_kernel<uint16_t, 128>), dim3((unsigned)grid), dim3(256), 0, s, p, bq, G);
    else hipLaunchKernelGGL((combine_kernel<uint16_t, 64>), dim3((unsigned)grid), dim3(256), 0, s, p, bq, G);
  } else {
    if (D == 128) hipLaunchKernelGGL((combine_kernel<float, 128>), dim3((unsigned)grid), dim3(256), 0, s, p, bq, G);
    else hipLaunchKernelGGL((combine_kernel<float, 64>), dim3((unsigned)grid), dim3(256), 0, s, p, bq, G);
  }
  return hipGetLastError();
}

}  // namespace minipic
