// Kernels around the flash loop: the KV-cache write, the cos/sin table and
// the merge of split tiles.
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
// Merge of split tiles: for every split (tile, KV head) group listed by
// plan_items, combine the pieces' partial results (O, m, l), m in log2 units,
// as O = sum_s 2^(m_s - m*) O_s / sum_s 2^(m_s - m*) l_s with m* = max_s m_s.
// One work-group unit is a block of RPW rows of one group; a row is handled
// by D/4 threads (4 elements each). The piece weights are computed lane-
// parallel (each lane owns pieces lane, lane + D/4, ...) into LDS, then the
// numerator sums the pieces in piece order with several loads in flight.
// The kernel also re-arms the attention scheduler's queue counters, which
// leaves the plan in the workspace ready for another attention run.
// ---------------------------------------------------------------------------
template <typename T, int D, int ROWS>
__global__ void __launch_bounds__(256) merge_kernel(AttnParams P, int G) {
  constexpr int TPR = D / 4;             // threads per row
  constexpr int RPW = 256 / TPR;         // rows per unit
  constexpr int NB = ROWS / RPW;         // units per group
  constexpr int KP = kMaxSplits / TPR;   // pieces per lane in the weight pass
  constexpr int UNR = 8;                 // pieces loaded together
  __shared__ float w_s[RPW][kMaxSplits];
  if (P.hdr->plan_key != P.plan_key) return;   // no plan of this run (uniform)
  // The attention kernel has finished (stream order): re-arm the scheduler's
  // counters, so that the plan serves the next run as well.
  if (blockIdx.x == 0 && threadIdx.x < kQueues) P.hdr->next[threadIdx.x] = first_tickets(P.num_wg, threadIdx.x);
  const int ngroups = (int)P.hdr->num_groups;
  const int r_in = threadIdx.x / TPR;
  const int d4 = threadIdx.x % TPR;
  for (int u = blockIdx.x; u < ngroups * NB; u += gridDim.x) {
    const Group grp = P.groups[u / NB];
    const TileDesc td = P.tiles[grp.tile];
    const int row = (u % NB) * RPW + r_in;
    const int tok = row / G;
    const bool valid = tok < td.nq && P.toks[(int64_t)grp.tile * (ROWS / G) + tok].c >= 0;
    const int ns = grp.nsplit;
    const int64_t base = (int64_t)grp.slot0 * ROWS + row;   // row of piece 0; piece s at + s * ROWS

    float m[KP], l[KP];
    float mstar = -INFINITY;
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int s = d4 + TPR * k;
      const float2 ml = s < ns ? P.part_ml[base + (int64_t)s * ROWS] : make_float2(-INFINITY, 0.f);
      m[k] = ml.x;
      l[k] = ml.y;
      mstar = fmaxf(mstar, ml.x);
    }
#pragma unroll
    for (int o = TPR / 2; o >= 1; o >>= 1) mstar = fmaxf(mstar, __shfl_xor(mstar, o, TPR));
    float den = 0.f;
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int s = d4 + TPR * k;
      const float w = m[k] == -INFINITY ? 0.f : exp2f(m[k] - mstar);
      if (s < ns) w_s[r_in][s] = w;
      den += w * l[k];
    }
#pragma unroll
    for (int o = TPR / 2; o >= 1; o >>= 1) den += __shfl_xor(den, o, TPR);
    __syncthreads();

    if (valid) {
      // elements d .. d+3 of the row in piece 0: the bf16 attention kernel
      // stores each 32-row block in its lanes' order ([d/32][(d%32)/8][lane][4],
      // lane = row % 32 + 32 ((d%8)/4)); the fp32 kernel stores plain rows
      const float* po;
      if constexpr (sizeof(T) == 2) {
        const int dg = d4 / 8, j = (d4 / 2) % 4, hh = d4 % 2;
        po = P.part_o + ((int64_t)grp.slot0 * ROWS + (row & ~31)) * D + ((dg * 4 + j) * 64 + (row & 31) + 32 * hh) * 4;
      } else {
        po = P.part_o + base * D + 4 * d4;
      }
      f32x4 num = {0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < ns; s0 += UNR) {
        f32x4 v[UNR];
#pragma unroll
        for (int k = 0; k < UNR; ++k)
          if (s0 + k < ns) v[k] = *(const f32x4*)(po + (int64_t)(s0 + k) * ROWS * D);
#pragma unroll
        for (int k = 0; k < UNR; ++k)
          if (s0 + k < ns) {
            const float w = w_s[r_in][s0 + k];
            if (w != 0.f) num += w * v[k];
          }
      }
      const float inv = 1.f / den;
      const int64_t qrow = (int64_t)td.row0 + tok;
      const int head = grp.g * G + row % G;
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
    __syncthreads();
  }
}

template <typename T, int D, int ROWS>
static void launch_merge_t(const AttnParams& p, int G, int max_groups, hipStream_t s) {
  constexpr int NB = ROWS / (256 / (D / 4));
  const int64_t units = (int64_t)max_groups * NB;
  const int grid = (int)(units < 4096 ? units : 4096);
  hipLaunchKernelGGL((merge_kernel<T, D, ROWS>), dim3(grid), dim3(256), 0, s, p, G);
}

hipError_t launch_merge(const AttnParams& p, int D, int dtype, int rows, int G, int max_groups, hipStream_t s) {
  if (dtype == MINIPIC_BF16) {
    if (rows == 256) {
      if (D == 128) launch_merge_t<uint16_t, 128, 256>(p, G, max_groups, s);
      else launch_merge_t<uint16_t, 64, 256>(p, G, max_groups, s);
    } else if (rows == 128) {
      if (D == 128) launch_merge_t<uint16_t, 128, 128>(p, G, max_groups, s);
      else launch_merge_t<uint16_t, 64, 128>(p, G, max_groups, s);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    if (D == 128) launch_merge_t<float, 128, 64>(p, G, max_groups, s);
    else launch_merge_t<float, 64, 64>(p, G, max_groups, s);
  }
  return hipGetLastError();
}

}  // namespace minipic
