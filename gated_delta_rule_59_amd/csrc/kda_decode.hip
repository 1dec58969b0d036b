// KDA decode step: one new token per (sequence, head), state updated in place.
//
// The work is one pass over the fixed-size state, independent of how many tokens came
// before (studioglobal.ai Kimi K3 pages: decode work does not grow with the context;
// orkas.ai infrastructure section: the state is updated in place). Per (n, h):
//     S' = Diag(exp g) S                (decay)
//     u  = v - S'^T k                   (prediction error of the decayed state)
//     S  = S' + beta k u^T              (delta-rule write)
//     o  = S^T q = S'^T q + beta (k.q) u
// so S is read once, two reductions over the key channels give S'^T k and S'^T q, and S
// is written once. HBM bound: 2 * 4 * dk * dv bytes of state per (n, h).
//
// One 256-thread workgroup per (n, h). Thread t owns value columns 4*(t % CG) .. +3
// (CG = DV / 4 column groups, one 16-byte vector) and key rows (t / CG) + RG * i,
// i < DK / RG (RG = 256 / CG row groups), so every wave reads whole 512-byte rows and the
// state stays in registers between the read and the write.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// At least 7 waves per SIMD (at most 72 VGPRs): more workgroups in flight per CU keep more
// of the state stream in flight. Measured on the 1 GiB decode workload: 0.378 ms per step,
// against 0.407 ms at the 95 VGPRs the compiler picks unconstrained and 0.390 ms at 6 waves;
// the 128 x 128 state then spills a few VGPRs, which costs less than the lost occupancy.
template <int DK, int DV, typename TIn, typename TOut>
__global__ __launch_bounds__(256, 7) void decode_step_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TIn* __restrict__ g, const TIn* __restrict__ beta, float* __restrict__ S,
    TOut* __restrict__ o, int64_t n_heads_total) {
  constexpr int CG = DV / 4;
  constexpr int RG = 256 / CG;
  constexpr int RPT = DK / RG;
  static_assert(RPT >= 1 && DK % RG == 0, "shape");

  const int64_t nh = blockIdx.x;  // (n * H + h)
  if (nh >= n_heads_total) return;
  const int t = threadIdx.x;
  const int cg = t % CG;
  const int rg = t / CG;

  __shared__ float s_k[DK], s_q[DK], s_d[DK];
  __shared__ float s_red[2][RG][DV];
  __shared__ float s_u[DV];

  const int64_t in_k = nh * DK;
  const int64_t in_v = nh * DV;
  __shared__ float s_kqp[4];
  float kq_part = 0.f;
  if (t < DK) {
    const float kc = ld(k, in_k + t), qc = ld(q, in_k + t);
    s_k[t] = kc;
    s_q[t] = qc;
    s_d[t] = __expf(ld(g, in_k + t));
    kq_part = kc * qc;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) kq_part += __shfl_xor(kq_part, m, 64);
  if ((t & 63) == 0) s_kqp[t >> 6] = kq_part;
  const float b = ld(beta, nh);

  floatx4* Sv = reinterpret_cast<floatx4*>(S + nh * (int64_t)DK * DV);
  floatx4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(&Sv[(rg + RG * i) * CG + cg]);
  __syncthreads();

  floatx4 pk = {0.f, 0.f, 0.f, 0.f}, pq = pk;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    const float d = s_d[r], kr = s_k[r], qr = s_q[r];
    s[i].x *= d; s[i].y *= d; s[i].z *= d; s[i].w *= d;
    pk.x += s[i].x * kr; pk.y += s[i].y * kr; pk.z += s[i].z * kr; pk.w += s[i].w * kr;
    pq.x += s[i].x * qr; pq.y += s[i].y * qr; pq.z += s[i].z * qr; pq.w += s[i].w * qr;
  }
  *reinterpret_cast<floatx4*>(&s_red[0][rg][4 * cg]) = pk;
  *reinterpret_cast<floatx4*>(&s_red[1][rg][4 * cg]) = pq;
  __syncthreads();

  if (t < DV) {
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      sk += s_red[0][r][t];
      sq += s_red[1][r][t];
    }
    const float u = ld(v, in_v + t) - sk;
    s_u[t] = u;
    const float kq = s_kqp[0] + s_kqp[1] + s_kqp[2] + s_kqp[3];
    st(o, in_v + t, sq + b * kq * u);
  }
  __syncthreads();

  const floatx4 u4 = *reinterpret_cast<const floatx4*>(&s_u[4 * cg]);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float bk = b * s_k[rg + RG * i];
    floatx4 w = s[i];
    w.x += bk * u4.x; w.y += bk * u4.y; w.z += bk * u4.z; w.w += bk * u4.w;
    __builtin_nontemporal_store(w, &Sv[(rg + RG * i) * CG + cg]);
  }
}

// Several tokens per (sequence, head) from one read of the state: speculative decoding
// evaluates m draft tokens without committing them, then commits the accepted prefix by
// replaying the same cached inputs (orkas.ai Kimi K3 page, serving-infrastructure section).
// Token j of sequence n sees the state after tokens 0..j-1 and itself; its output is written
// when o is given. With accept == nullptr the state is left as it was (verification); with
// accept, S[n] becomes the state after the first clamp(accept[n], 0, m) tokens. The state
// stays in registers across the tokens: one read of S, and one write only when committing.
// Same thread layout as decode_step_kernel; inputs are [N, m, H, d].
// At least 4 waves per SIMD (128 VGPRs): verification of 4 drafts on the 1 GiB decode state
// takes 0.264 ms against 0.296 ms at the 140 VGPRs the compiler picks unconstrained.
template <int DK, int DV, typename TIn, typename TOut>
__global__ __launch_bounds__(256, 4) void decode_multi_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TIn* __restrict__ g, const TIn* __restrict__ beta, float* __restrict__ S,
    TOut* __restrict__ o, const int32_t* __restrict__ accept, int H, int m,
    int64_t n_heads_total) {
  constexpr int CG = DV / 4;
  constexpr int RG = 256 / CG;
  constexpr int RPT = DK / RG;
  static_assert(RPT >= 1 && DK % RG == 0, "shape");

  const int64_t nh = blockIdx.x;  // (n * H + h)
  if (nh >= n_heads_total) return;
  const int64_t n = nh / H, h = nh % H;
  const int t = threadIdx.x;
  const int cg = t % CG;
  const int rg = t / CG;
  const int keep = accept ? min(max(accept[n], 0), m) : 0;  // tokens committed to S
  const int upto = o ? m : keep;                             // tokens evaluated

  __shared__ float s_k[DK], s_q[DK], s_d[DK];
  __shared__ float s_red[2][RG][DV];
  __shared__ float s_u[DV];
  __shared__ float s_kqp[4];

  floatx4* Sv = reinterpret_cast<floatx4*>(S + nh * (int64_t)DK * DV);
  floatx4 s[RPT];
  if (upto > 0) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(&Sv[(rg + RG * i) * CG + cg]);
  }
  for (int j = 0; j < upto; ++j) {
    const int64_t tok = (n * m + j) * H + h;  // row of token j of this (sequence, head)
    const int64_t in_k = tok * DK, in_v = tok * DV;
    __syncthreads();  // the previous token's reads of s_k, s_u are done
    float kq_part = 0.f;
    if (t < DK) {
      const float kc = ld(k, in_k + t), qc = ld(q, in_k + t);
      s_k[t] = kc;
      s_q[t] = qc;
      s_d[t] = __expf(ld(g, in_k + t));
      kq_part = kc * qc;
    }
#pragma unroll
    for (int mm = 32; mm >= 1; mm >>= 1) kq_part += __shfl_xor(kq_part, mm, 64);
    if ((t & 63) == 0) s_kqp[t >> 6] = kq_part;
    const float b = ld(beta, tok);
    __syncthreads();

    floatx4 pk = {0.f, 0.f, 0.f, 0.f}, pq = pk;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + RG * i;
      const float d = s_d[r], kr = s_k[r], qr = s_q[r];
      s[i].x *= d; s[i].y *= d; s[i].z *= d; s[i].w *= d;
      pk.x += s[i].x * kr; pk.y += s[i].y * kr; pk.z += s[i].z * kr; pk.w += s[i].w * kr;
      pq.x += s[i].x * qr; pq.y += s[i].y * qr; pq.z += s[i].z * qr; pq.w += s[i].w * qr;
    }
    *reinterpret_cast<floatx4*>(&s_red[0][rg][4 * cg]) = pk;
    *reinterpret_cast<floatx4*>(&s_red[1][rg][4 * cg]) = pq;
    __syncthreads();

    if (t < DV) {
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        sk += s_red[0][r][t];
        sq += s_red[1][r][t];
      }
      const float u = ld(v, in_v + t) - sk;
      s_u[t] = u;
      const float kq = s_kqp[0] + s_kqp[1] + s_kqp[2] + s_kqp[3];
      if (o) st(o, in_v + t, sq + b * kq * u);
    }
    __syncthreads();

    const floatx4 u4 = *reinterpret_cast<const floatx4*>(&s_u[4 * cg]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float bk = b * s_k[rg + RG * i];
      s[i].x += bk * u4.x; s[i].y += bk * u4.y; s[i].z += bk * u4.z; s[i].w += bk * u4.w;
    }
    if (j + 1 == keep) {  // the accepted prefix ends here: commit
#pragma unroll
      for (int i = 0; i < RPT; ++i) __builtin_nontemporal_store(s[i], &Sv[(rg + RG * i) * CG + cg]);
    }
  }
}

template <int DK, int DV, typename TIn, typename TOut>
static hipError_t launch_decode_multi_t(const DecodeMultiPlan& p, hipStream_t stream) {
  const int64_t nh = (int64_t)p.N * p.H;
  hipLaunchKernelGGL((decode_multi_kernel<DK, DV, TIn, TOut>), dim3((unsigned)nh), dim3(256), 0,
                     stream, static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k),
                     static_cast<const TIn*>(p.v), static_cast<const TIn*>(p.g),
                     static_cast<const TIn*>(p.beta), p.S, static_cast<TOut*>(p.o), p.accept,
                     p.H, p.m, nh);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_decode_multi_d(const DecodeMultiPlan& p, hipStream_t stream) {
  if (p.act_bf16)
    return p.out_bf16 ? launch_decode_multi_t<DK, DV, uint16_t, uint16_t>(p, stream)
                      : launch_decode_multi_t<DK, DV, uint16_t, float>(p, stream);
  return p.out_bf16 ? launch_decode_multi_t<DK, DV, float, uint16_t>(p, stream)
                    : launch_decode_multi_t<DK, DV, float, float>(p, stream);
}

hipError_t launch_decode_multi(const DecodeMultiPlan& p, hipStream_t stream) {
#define KDA_DECODE_CASE(A, B) \
  if (p.dk == A && p.dv == B) return launch_decode_multi_d<A, B>(p, stream);
  KDA_DECODE_CASE(32, 32) KDA_DECODE_CASE(32, 64) KDA_DECODE_CASE(32, 128)
  KDA_DECODE_CASE(64, 32) KDA_DECODE_CASE(64, 64) KDA_DECODE_CASE(64, 128)
  KDA_DECODE_CASE(128, 32) KDA_DECODE_CASE(128, 64) KDA_DECODE_CASE(128, 128)
#undef KDA_DECODE_CASE
  return hipErrorInvalidValue;
}

template <int DK, int DV, typename TIn, typename TOut>
static hipError_t launch_decode_t(const DecodePlan& p, hipStream_t stream) {
  const int64_t nh = (int64_t)p.N * p.H;
  hipLaunchKernelGGL((decode_step_kernel<DK, DV, TIn, TOut>), dim3((unsigned)nh), dim3(256), 0,
                     stream, static_cast<const TIn*>(p.q), static_cast<const TIn*>(p.k),
                     static_cast<const TIn*>(p.v), static_cast<const TIn*>(p.g),
                     static_cast<const TIn*>(p.beta), p.S, static_cast<TOut*>(p.o), nh);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_decode_d(const DecodePlan& p, hipStream_t stream) {
  if (p.act_bf16)
    return p.out_bf16 ? launch_decode_t<DK, DV, uint16_t, uint16_t>(p, stream)
                      : launch_decode_t<DK, DV, uint16_t, float>(p, stream);
  return p.out_bf16 ? launch_decode_t<DK, DV, float, uint16_t>(p, stream)
                    : launch_decode_t<DK, DV, float, float>(p, stream);
}

hipError_t launch_decode(const DecodePlan& p, hipStream_t stream) {
#define KDA_DECODE_CASE(A, B) \
  if (p.dk == A && p.dv == B) return launch_decode_d<A, B>(p, stream);
  KDA_DECODE_CASE(32, 32) KDA_DECODE_CASE(32, 64) KDA_DECODE_CASE(32, 128)
  KDA_DECODE_CASE(64, 32) KDA_DECODE_CASE(64, 64) KDA_DECODE_CASE(64, 128)
  KDA_DECODE_CASE(128, 32) KDA_DECODE_CASE(128, 64) KDA_DECODE_CASE(128, 128)
#undef KDA_DECODE_CASE
  return hipErrorInvalidValue;
}

}  // namespace kda
