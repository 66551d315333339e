// fp32 position-free paged prefill attention (vector ALU).
//
// Same method and work decomposition as the bf16 MFMA kernel ("MiniPIC:
// Flexible Position-Independent Caching in <100LOC", §3.2.1 score equation,
// §3.2.2 in-kernel rotation of each K tile after a cos/sin lookup at pi(j)),
// for float32 caches: rows of 4 lanes each own a quarter of the head dim,
// K tiles of one cache block are rotated in fp32 while staged through LDS,
// and an exact online softmax runs per key. It serves fp32 models and small
// shapes; bf16 work goes to the MFMA kernel.
#include "common.h"

namespace minipic {

constexpr int kNTf = 256;
constexpr int kRowsF = 64;   // 4 lanes per row

template <int D, int G, bool ROPE>
__global__ void __launch_bounds__(kNTf) attn_f32_kernel(AttnParams P) {
  constexpr int BQ = kRowsF / G;
  constexpr int DQ = D / 4;
  __shared__ PlanSmem<BQ> sm;
  __shared__ float kt[kBlock][D + 1];
  __shared__ float vt[kBlock][D + 1];

  TileInfo t;
  decode_block(P, blockIdx.x, t);
  if (!plan_tile<kNTf, BQ>(P, t, sm)) return;

  const int tid = threadIdx.x;
  const int row = tid >> 2;
  const int qd = (tid & 3) * DQ;      // this lane's slice of the head dim
  const int tok = row / G;
  const int head = t.g * G + row % G;
  const bool rvalid = tok < t.nq && sm.qctx[tok] >= 0;
  const int c_row = rvalid ? sm.qctx[tok] : -1;
  const int ent = rvalid ? sm.qent[tok] : 0;
  const int bq_row = rvalid ? sm.e_bq[ent] : -1;
  const int span_row = rvalid ? sm.e_span[ent] : 0;
  const bool pdep_row = rvalid && sm.e_pdep[ent];
  const int64_t qrow = (int64_t)t.row0 + tok;
  const int32_t* lpos = P.logical_pos + (int64_t)t.r * P.max_blocks * kBlock;

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
  const float sl2 = P.scale_log2;
  const float* kc = (const float*)P.k_cache;
  const float* vc = (const float*)P.v_cache;

  for (int c0 = t.p0; c0 < t.p1; c0 += kListMax) {
    const int c1 = min(t.p1, c0 + kListMax);
    const int n_l = build_list<kNTf, BQ>(P, t, sm, c0, c1);
    for (int e = 0; e < n_l; ++e) {
      const int ph = sm.l_phys[e];
      const int kbk = sm.l_kb[e];
      // stage the rotated K block and V block (transposed back to [key][d])
      for (int u = tid; u < kBlock * (D / 2); u += kNTf) {
        const int key = u / (D / 2);
        const int i = u % (D / 2);
        float a = 0.f, b = 0.f;
        if (ph >= 0) {
          const float* kr = kc + (((int64_t)ph * P.hkv + t.g) * kBlock + key) * D;
          a = kr[i];
          b = kr[i + D / 2];
          if (ROPE) {
            int pos = lpos[kbk * kBlock + key];
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
        vt[key][d] = ph >= 0 ? vc[(((int64_t)ph * P.hkv + t.g) * D + d) * kBlock + key] : 0.f;
      }
      __syncthreads();
      const int spk = sm.l_span[e];
      const int flk = sm.l_flags[e];
      const bool vis = rvalid && kbk <= bq_row &&
                       (pdep_row || (flk & MINIPIC_BLK_GLOBAL) || spk == span_row);
      for (int key = 0; key < kBlock; ++key) {
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < DQ; ++i) dot = fmaf(qv[i], kt[key][qd + i], dot);
        dot += __shfl_xor(dot, 1, 64);
        dot += __shfl_xor(dot, 2, 64);
        if (vis && kbk * kBlock + key <= c_row) {
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

  if (!rvalid) return;
  if (t.nsplit == 1) {
    float* op = (float*)P.out + (qrow * P.hq + head) * D + qd;
    const float inv = 1.f / l_run;
#pragma unroll
    for (int i = 0; i < DQ; ++i) op[i] = o[i] * inv;
  } else {
    const int64_t pr = ((int64_t)t.s * P.total_q + qrow) * P.hq + head;
    float* op = P.part_o + pr * D + qd;
#pragma unroll
    for (int i = 0; i < DQ; ++i) op[i] = o[i];
    if ((tid & 3) == 0) P.part_ml[pr] = make_float2(m_run, l_run);
  }
}

template <int D, int G, bool ROPE>
static hipError_t launch_one_f(const AttnParams& p, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_f32_kernel<D, G, ROPE>), dim3((unsigned)grid), dim3(kNTf), 0, s, p);
  return hipGetLastError();
}

template <int D, bool ROPE>
static hipError_t launch_gf(const AttnParams& p, int G, int64_t grid, hipStream_t s) {
  switch (G) {
    case 1: return launch_one_f<D, 1, ROPE>(p, grid, s);
    case 2: return launch_one_f<D, 2, ROPE>(p, grid, s);
    case 4: return launch_one_f<D, 4, ROPE>(p, grid, s);
    case 8: return launch_one_f<D, 8, ROPE>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_f32(const AttnParams& p, int D, int G, bool rope, int64_t grid, hipStream_t s) {
  if (D == 128) return rope ? launch_gf<128, true>(p, G, grid, s) : launch_gf<128, false>(p, G, grid, s);
  if (D == 64) return rope ? launch_gf<64, true>(p, G, grid, s) : launch_gf<64, false>(p, G, grid, s);
  return hipErrorInvalidValue;
}

}  // namespace minipic
