// fp32 position-free paged prefill attention (vector ALU).
//
// Same method and work items as the bf16 MFMA kernel ("MiniPIC: Flexible
// Position-Independent Caching in <100LOC", §3.2.1 score equation, §3.2.2
// in-kernel rotation of each K tile after a cos/sin lookup at pi(j)), for
// float32 caches: rows of 4 lanes each own a quarter of the head dim, K tiles
// of one cache block are rotated in fp32 while staged through LDS, and an
// exact online softmax runs per key. It serves fp32 models and small shapes;
// bf16 work goes to the MFMA kernel.
#include "common.h"

namespace minipic {

constexpr int kNTf = 256;
constexpr int kRowsF = 64;        // 4 lanes per row
constexpr int kListMaxF = 256;

template <int D, int G, bool ROPE>
__global__ void __launch_bounds__(kNTf) attn_f32_kernel(AttnParams P) {
  constexpr int BQ = kRowsF / G;
  constexpr int DQ = D / 4;
  __shared__ BlkDesc lst[kListMaxF];
  __shared__ int s_next;
  __shared__ uint32_t s_qs[kQueues], s_qc[kQueues];
  __shared__ float kt[kBlock][D + 1];
  __shared__ float vt[kBlock][D + 1];

  const int tid = threadIdx.x;
  const int row = tid >> 2;
  const int qd = (tid & 3) * DQ;      // this lane's slice of the head dim
  const int tok = row / G;
  const int hig = row % G;
  const float sl2 = P.scale_log2;
  const float* kc = (const float*)P.k_cache;
  const float* vc = (const float*)P.v_cache;
  // a run needs the plan of its own configuration in the workspace
  if (P.hdr->plan_key != P.plan_key) {   // uniform (one scalar load)
    if (blockIdx.x == 0 && tid == 0) atomicOr(P.err, (uint32_t)MINIPIC_EW_PLAN);
    return;
  }
  if (tid < kQueues) {
    s_qs[tid] = P.hdr->qstart[tid];
    s_qc[tid] = P.hdr->qcount[tid];
  }
  int q_cur = blockIdx.x % kQueues;   // queue being drained (thread 0)
  __syncthreads();
  // the first item is the work-group's own ticket (the planner starts each
  // queue's counter past the work-groups that drain it)
  if (tid == 0) s_next = resolve_ticket(P.hdr, s_qs, s_qc, q_cur, blockIdx.x / kQueues);
  __syncthreads();
  int it = __builtin_amdgcn_readfirstlane(s_next);
  while (it >= 0) {
    uint32_t ticket = 0;   // claim of the following item, checked when this one ends
    if (tid == 0) ticket = atomicAdd(&P.hdr->next[q_cur], 1u);
    const Item item = P.items[it];
    const int g = item.gsn & 0xff;
    const int sp = (item.gsn >> 8) & 0xfff;
    const int ns = item.gsn >> 20;
    const TokDesc tk = P.toks[(int64_t)item.tile * BQ + tok];
    const bool rvalid = tok < item.nq && tk.c >= 0;
    const int c_row = rvalid ? tk.c : -1;
    const int bq_row = rvalid ? (c_row >> 4) : -1;
    const int span_row = tk.span;
    const int lo_row = tk.lo;
    const bool pdep_row = rvalid && tk.pdep;
    const int head = g * G + hig;
    const int64_t qrow = (int64_t)item.row0 + tok;
    const int32_t* lpos = P.logical_pos + (int64_t)item.r * P.max_blocks * kBlock;
    const BlkDesc* blist = P.blist + (int64_t)item.tile * P.max_blocks;

    // query slice; with MINIPIC_FLAG_ROTATE_Q the rotate-half partner of
    // element i is i + D/2, which lives in lane (tid ^ 2)
    float qv[DQ];
    {
      const float* qp = (const float*)P.q + (qrow * P.hq + head) * D + qd;
#pragma unroll
      for (int i = 0; i < DQ; ++i) qv[i] = rvalid ? qp[i] : 0.f;
      if (P.flags & MINIPIC_FLAG_ROTATE_Q) {
        int pos = rvalid ? lpos[c_row] : 0;
        if (pos < 0 || pos >= P.max_pos) {
          atomicOr(P.err, (uint32_t)MINIPIC_EW_POS);
          pos = pos < 0 ? 0 : P.max_pos - 1;
        }
        const float* cs = P.cos_sin + (int64_t)pos * D;
        const bool first_half = qd < D / 2;
#pragma unroll
        for (int i = 0; i < DQ; ++i) {
          const float partner = __shfl_xor(qv[i], 2, 64);
          const int fi = (qd + i) % (D / 2);
          const float c = cs[fi], s = cs[D / 2 + fi];
          qv[i] = first_half ? qv[i] * c - partner * s : qv[i] * c + partner * s;
        }
      }
    }
    float o[DQ];
#pragma unroll
    for (int i = 0; i < DQ; ++i) o[i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    for (int c0 = item.p0; c0 < item.p1; c0 += kListMaxF) {
      const int n_l = min(kListMaxF, item.p1 - c0);
      for (int i = tid; i < n_l; i += kNTf) lst[i] = blist[c0 + i];
      __syncthreads();
      for (int e = 0; e < n_l; ++e) {
        const BlkDesc bd = lst[e];
        // stage the rotated K block and V block (transposed back to [key][d])
        for (int u = tid; u < kBlock * (D / 2); u += kNTf) {
          const int key = u / (D / 2);
          const int i = u % (D / 2);
          float a = 0.f, b = 0.f;
          if (bd.phys >= 0) {
            const float* kr = kc + (((int64_t)bd.phys * P.hkv + g) * kBlock + key) * D;
            a = kr[i];
            b = kr[i + D / 2];
            if (ROPE) {
              // a key past the context holds no token (never visible): any table row will do
              int pos = key >= bd.nvalid ? 0 : (bd.pos0 >= 0 ? bd.pos0 + key : lpos[bd.kb * kBlock + key]);
              if (pos < 0 || pos >= P.max_pos) {
                atomicOr(P.err, (uint32_t)MINIPIC_EW_POS);
                pos = pos < 0 ? 0 : P.max_pos - 1;
              }
              const float c = P.cos_sin[(int64_t)pos * D + i];
              const float s = P.cos_sin[(int64_t)pos * D + D / 2 + i];
              const float ra = a * c - b * s;
              const float rb = b * c + a * s;
              a = ra;
              b = rb;
            }
          }
          kt[key][i] = a;
          kt[key][i + D / 2] = b;
        }
        for (int u = tid; u < kBlock * D; u += kNTf) {
          const int d = u / kBlock;
          const int key = u % kBlock;
          vt[key][d] = bd.phys >= 0 ? vc[(((int64_t)bd.phys * P.hkv + g) * D + d) * kBlock + key] : 0.f;
        }
        __syncthreads();
        const bool vis = rvalid && block_visible(bd.kb, bd.span, bd.flags, bq_row, span_row, pdep_row, lo_row);
        for (int key = 0; key < kBlock; ++key) {
          float dot = 0.f;
#pragma unroll
          for (int i = 0; i < DQ; ++i) dot = fmaf(qv[i], kt[key][qd + i], dot);
          dot += __shfl_xor(dot, 1, 64);
          dot += __shfl_xor(dot, 2, 64);
          if (vis && bd.kb * kBlock + key <= c_row) {
            const float x = dot * sl2;
            const float m_new = fmaxf(m_run, x);
            const float corr = exp2f(m_run - m_new);
            const float p = exp2f(x - m_new);
            l_run = l_run * corr + p;
#pragma unroll
            for (int i = 0; i < DQ; ++i) o[i] = o[i] * corr + p * vt[key][qd + i];
            m_run = m_new;
          }
        }
        __syncthreads();
      }
    }

    float* op = (float*)P.out + (qrow * P.hq + head) * D + qd;
    if (ns == 1) {
      if (rvalid) {
        const float inv = 1.f / l_run;
#pragma unroll
        for (int i = 0; i < DQ; ++i) op[i] = o[i] * inv;
      }
    } else if (rvalid) {
      // a piece of a split tile: fp32 partial result to its slot (merged by merge_kernel)
      const int64_t pr = (int64_t)(item.slot0 + g * ns + sp) * kRowsF + row;
      float* po = P.part_o + pr * D + qd;
#pragma unroll
      for (int i = 0; i < DQ; ++i) po[i] = o[i];
      if ((tid & 3) == 0) P.part_ml[pr] = make_float2(m_run, l_run);
    }
    if (tid == 0) s_next = resolve_ticket(P.hdr, s_qs, s_qc, q_cur, ticket);
    __syncthreads();
    // s_next is written again only after the next item's barriers
    it = __builtin_amdgcn_readfirstlane(s_next);
  }
}

template <int D, int G, bool ROPE>
static hipError_t launch_one_f(const AttnParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_f32_kernel<D, G, ROPE>), dim3((unsigned)grid), dim3(kNTf), 0, s, p);
  return hipGetLastError();
}

template <int D, bool ROPE>
static hipError_t launch_gf(const AttnParams& p, int G, int grid, hipStream_t s) {
  switch (G) {
    case 1: return launch_one_f<D, 1, ROPE>(p, grid, s);
    case 2: return launch_one_f<D, 2, ROPE>(p, grid, s);
    case 4: return launch_one_f<D, 4, ROPE>(p, grid, s);
    case 8: return launch_one_f<D, 8, ROPE>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_f32(const AttnParams& p, int D, int G, bool rope, int grid, hipStream_t s) {
  if (D == 128) return rope ? launch_gf<128, true>(p, G, grid, s) : launch_gf<128, false>(p, G, grid, s);
  if (D == 64) return rope ? launch_gf<64, true>(p, G, grid, s) : launch_gf<64, false>(p, G, grid, s);
  return hipErrorInvalidValue;
}

int attn_f32_blocks_per_cu(int D, int G, bool rope) {
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
#define MINIPIC_OCC(DD, GG, RR)                                                                   \
  if (D == DD && G == GG && rope == RR)                                                          \
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_f32_kernel<DD, GG, RR>, kNTf, 0);
  MINIPIC_OCC(128, 1, true) MINIPIC_OCC(128, 2, true) MINIPIC_OCC(128, 4, true) MINIPIC_OCC(128, 8, true)
  MINIPIC_OCC(128, 1, false) MINIPIC_OCC(128, 2, false) MINIPIC_OCC(128, 4, false) MINIPIC_OCC(128, 8, false)
  MINIPIC_OCC(64, 1, true) MINIPIC_OCC(64, 2, true) MINIPIC_OCC(64, 4, true) MINIPIC_OCC(64, 8, true)
  MINIPIC_OCC(64, 1, false) MINIPIC_OCC(64, 2, false) MINIPIC_OCC(64, 4, false) MINIPIC_OCC(64, 8, false)
#undef MINIPIC_OCC
  return (e == hipSuccess && n > 0) ? n : 1;
}

}  // namespace minipic
