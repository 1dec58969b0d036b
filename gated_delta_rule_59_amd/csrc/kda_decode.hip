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
#include <type_traits>

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
// Same thread layout as decode_step_kernel; inputs are [N, m, H, d]. This token loop serves a
// single draft, more than eight, and head sizes other than 128; draft_chunk_kernel below
// takes 2..8 drafts at dk = dv = 128 in one pass.
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

// Several drafts as one mini-chunk of the chunked form (the same algebra the prefill uses for
// its 64-token chunks). For tokens i < m of (n, h) entering with state S, per key channel c:
//   d_i = e^{g_i},  Gam_i = d_0 ... d_i,  P(l, i) = d_{l+1} ... d_i  (P(i, i) = 1)
//   state before token i's write:  Diag(Gam_i) S + sum_{l<i} Diag(P(l, i)) b_l k_l u_l^T, so
//   u_i = v_i - S^T (Gam_i k_i) - sum_{l<i} A_il u_l,   A_il = b_l sum_c k_ic k_lc P(l, i)_c
//   o_j = S^T (Gam_j q_j) + sum_{i<=j} B_ji u_i,          B_ji = b_i sum_c q_jc k_ic P(i, j)_c
//   state after the first a tokens:  Diag(Gam_{a-1}) S + sum_{l<a} Diag(P(l, a-1)) b_l k_l u_l^T
// The state enters only through the 2m column reductions S^T (Gam_i k_i) and S^T (Gam_j q_j):
// one pass over S serves every draft, a verification streams S through 2m accumulators per
// column and holds none of it, and a commit keeps its slice of S in registers for the one
// update with all accepted tokens. M >= m is the register size (missing tokens are zero).
//
// Thread t of wave w owns value columns 2 (t & 63), +1 and key rows w + 4 i (i < 32): every
// load is one 512-byte row per wave, and the column partial sums of a wave need no exchange
// between its lanes. Verification and commit share every instruction that forms the outputs,
// written as explicit fused multiply-adds in a fixed order, so a commit call writes outputs
// bitwise equal to those of the verification call with the same inputs.
typedef float floatx2 __attribute__((ext_vector_type(2)));

// Sum over the 16 lanes of a DPP row, left in the row's last lane (inclusive scan, zero fill).
__device__ __forceinline__ float dpp_row_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
  return x;
}

// Occupancy (waves per SIMD) on the 1 GiB decode state with four drafts: a verification at 6
// (72 VGPRs; 0.187 ms, against 0.187 at 7 and 0.189 at 8), a commit at 4 (the 128 x 128
// state held in 64 VGPRs; 0.381 ms, against 0.390 at 5). Eight drafts fit 3 workgroups per CU
// in LDS.
template <int M, bool COMMIT, bool OUT, typename TIn, typename TOut>
__global__ __launch_bounds__(256, M > 4 ? 3 : (COMMIT ? 4 : 6)) void draft_chunk_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TIn* __restrict__ g, const TIn* __restrict__ beta, float* __restrict__ S,
    TOut* __restrict__ o, const int32_t* __restrict__ accept, int H, int m,
    int64_t n_heads_total) {
  constexpr int DK = 128, DV = 128;
  constexpr int RPT = DK / 4;  // rows per thread
  constexpr int WIN = 8;       // rows in flight per thread while verifying
  constexpr int NAB = M * M;   // A_il at [i][l] (l < i), B_ji at [i][j] (i <= j)
  constexpr int NT = OUT ? 2 * M : M;  // reductions: S^T (Gam_i k_i), then S^T (Gam_j q_j)
  static_assert(M % 4 == 0 && RPT % WIN == 0 && (COMMIT || OUT), "shape");

  const int64_t nh = blockIdx.x;  // (n * H + h)
  if (nh >= n_heads_total) return;
  const int64_t n = nh / H, h = nh % H;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int a = COMMIT ? min(max(accept[n], 0), m) : 0;  // tokens committed to S

  __shared__ __align__(16) float s_tab[DK][NT];      // row c: Gam_i k_ic (i < M), Gam_j q_jc
  __shared__ __align__(16) float s_red[4][NT][DV];   // per-wave column sums
  __shared__ float s_part[8][NAB];                      // 16-channel partial sums of A, B
  __shared__ float s_ab[NAB];
  __shared__ __align__(16) float s_cf[COMMIT ? DK : 1][M];  // b_l k_lc P(l, a-1)_c, l < a
  __shared__ float s_gam[COMMIT ? DK : 1];                  // Gam_{a-1}
  __shared__ __align__(16) float s_u[COMMIT ? M : 1][DV];

  // ---- the drafts' inputs first (threads 0..127 own key channel c = t, and value column t):
  //      loads complete in issue order, so the work on them below waits for these loads only,
  //      not for the state behind them
  float kk[M], qq[M], dd[M], bb[M], vv[M];
#pragma unroll
  for (int i = 0; i < M; ++i) kk[i] = qq[i] = dd[i] = bb[i] = vv[i] = 0.f;
  if (t < DK) {
#pragma unroll
    for (int i = 0; i < M; ++i) {
      if (i < m) {
        const int64_t tok = (n * m + i) * H + h;
        kk[i] = ld(k, tok * DK + t);
        qq[i] = ld(q, tok * DK + t);
        dd[i] = ld(g, tok * DK + t);
        bb[i] = ld(beta, tok);
        vv[i] = ld(v, tok * DV + t);
      }
    }
  }
  const floatx2* Sv = reinterpret_cast<const floatx2*>(S + nh * (int64_t)DK * DV);
  auto s_ptr = [&](int i) { return &Sv[(w + 4 * i) * (DV / 2) + lane]; };
  floatx2 s[COMMIT ? RPT : WIN];
#pragma unroll
  for (int i = 0; i < (COMMIT ? RPT : WIN); ++i) s[i] = __builtin_nontemporal_load(s_ptr(i));

  // ---- per key channel (threads 0..127): decay products, the reduction tables, the terms
  //      of A and B, and (commit) the update coefficients
  if (t < DK) {
    const int c = t;
#pragma unroll
    for (int i = 0; i < M; ++i) dd[i] = i < m ? __expf(dd[i]) : 1.f;  // e^{g_i}; 1 past the drafts
    float tk[M], tq[M];
    float gam = 1.f;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      gam = gam * dd[i];
      tk[i] = gam * kk[i];
      tq[i] = gam * qq[i];
      if (COMMIT && i == a - 1) s_gam[c] = gam;
    }
#pragma unroll
    for (int i = 0; i < M; i += 4) {
      *reinterpret_cast<floatx4*>(&s_tab[c][i]) = floatx4{tk[i], tk[i + 1], tk[i + 2], tk[i + 3]};
      if (OUT)
        *reinterpret_cast<floatx4*>(&s_tab[c][M + i]) = floatx4{tq[i], tq[i + 1], tq[i + 2], tq[i + 3]};
    }
    // terms: pair (l, i), l <= i, with P = P(l, i)
    float cf[M];
#pragma unroll
    for (int i = 0; i < M; ++i) cf[i] = 0.f;
#pragma unroll
    for (int l = 0; l < M; ++l) {
      float P = 1.f;
#pragma unroll
      for (int i = l; i < M; ++i) {
        if (i > l) P = P * dd[i];
        if (COMMIT && i == a - 1) cf[l] = (bb[l] * kk[l]) * P;
        const float kp = kk[l] * P;
        float ta = 0.f, tb = 0.f;
        if (i > l) ta = dpp_row_sum(kk[i] * kp);  // A_il / b_l
        if (OUT) tb = dpp_row_sum(qq[i] * kp);     // B_il / b_l (token i's output, draft l)
        if ((lane & 15) == 15) {
          if (i > l) s_part[4 * w + (lane >> 4)][i * M + l] = ta;
          if (OUT) s_part[4 * w + (lane >> 4)][l * M + i] = tb;
        }
      }
    }
    if (COMMIT) {
#pragma unroll
      for (int i = 0; i < M; i += 4)
        *reinterpret_cast<floatx4*>(&s_cf[c][i]) = floatx4{cf[i], cf[i + 1], cf[i + 2], cf[i + 3]};
    }
  }
  __syncthreads();
  if (t < NAB && (OUT || t % M < t / M)) {  // (r, c): A_rc = b_c sum (c < r), B_cr = b_r sum (r <= c)
    const int r = t / M, cc = t % M;
    float sum = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) sum += s_part[p][t];
    const int bi = cc < r ? cc : r;  // the draft whose b scales the entry (0 past the drafts)
    float b = 0.f;
#pragma unroll
    for (int i = 0; i < M; ++i) b = i == bi ? bb[i] : b;
    s_ab[t] = sum * b;
  }

  // ---- one pass over S: the 2M column reductions of this thread's rows
  floatx2 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = floatx2{0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const floatx2 x = s[COMMIT ? i : i % WIN];
    if (!COMMIT && i + WIN < RPT) s[i % WIN] = __builtin_nontemporal_load(s_ptr(i + WIN));
    const float* tr = s_tab[w + 4 * i];
#pragma unroll
    for (int j = 0; j < NT; j += 4) {
      const floatx4 f = *reinterpret_cast<const floatx4*>(tr + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[j + e].x = fmaf(x.x, f[e], acc[j + e].x);
        acc[j + e].y = fmaf(x.y, f[e], acc[j + e].y);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) *reinterpret_cast<floatx2*>(&s_red[w][j][2 * lane]) = acc[j];
  __syncthreads();

  // ---- per value column (threads 0..127): the triangular solve for u, then the outputs
  if (t < DV) {
    const int c = t;
    float u[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const float rk = ((s_red[0][i][c] + s_red[1][i][c]) + s_red[2][i][c]) + s_red[3][i][c];
      float x = vv[i] - rk;
#pragma unroll
      for (int l = 0; l < i; ++l) x = fmaf(-s_ab[i * M + l], u[l], x);
      u[i] = x;
      if (COMMIT) s_u[i][c] = x;
    }
    if (OUT) {
#pragma unroll
      for (int j = 0; j < M; ++j) {
        if (j >= m) break;
        float y = ((s_red[0][M + j][c] + s_red[1][M + j][c]) + s_red[2][M + j][c]) + s_red[3][M + j][c];
#pragma unroll
        for (int i = 0; i <= j; ++i) y = fmaf(s_ab[i * M + j], u[i], y);
        st(o, ((n * m + j) * H + h) * DV + c, y);
      }
    }
  }
  if constexpr (COMMIT) {
    __syncthreads();
    if (a > 0) {
      // rejected drafts get u = 0 as well as a zero coefficient, so that whatever their
      // inputs hold adds nothing
      floatx2 ul[M];
#pragma unroll
      for (int l = 0; l < M; ++l)
        ul[l] = l < a ? *reinterpret_cast<const floatx2*>(&s_u[l][2 * lane]) : floatx2{0.f, 0.f};
      floatx2* Sw = reinterpret_cast<floatx2*>(S + nh * (int64_t)DK * DV);
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = w + 4 * i;
        const float gm = s_gam[r];
        floatx2 x = {s[i].x * gm, s[i].y * gm};
#pragma unroll
        for (int l = 0; l < M; l += 4) {
          const floatx4 cl = *reinterpret_cast<const floatx4*>(&s_cf[r][l]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x.x = fmaf(cl[e], ul[l + e].x, x.x);
            x.y = fmaf(cl[e], ul[l + e].y, x.y);
          }
        }
        __builtin_nontemporal_store(x, &Sw[r * (DV / 2) + lane]);
      }
    }
  }
}

template <int DK, int DV, typename TIn, typename TOut>
static hipError_t launch_decode_multi_t(const DecodeMultiPlan& p, hipStream_t stream) {
  const int64_t nh = (int64_t)p.N * p.H;
  const TIn *q = static_cast<const TIn*>(p.q), *k = static_cast<const TIn*>(p.k),
            *v = static_cast<const TIn*>(p.v), *g = static_cast<const TIn*>(p.g),
            *beta = static_cast<const TIn*>(p.beta);
  TOut* o = static_cast<TOut*>(p.o);
  if constexpr (DK == 128 && DV == 128) {
    // 2..8 drafts: one pass over S (a single token, and longer drafts, take the token loop)
    if (p.m >= 2 && p.m <= 8) {
      auto pick = [&](auto M) {
        constexpr int Mv = decltype(M)::value;
        return !p.accept ? draft_chunk_kernel<Mv, false, true, TIn, TOut>
               : o       ? draft_chunk_kernel<Mv, true, true, TIn, TOut>
                         : draft_chunk_kernel<Mv, true, false, TIn, TOut>;
      };
      auto kern = p.m <= 4 ? pick(std::integral_constant<int, 4>{})
                           : pick(std::integral_constant<int, 8>{});
      hipLaunchKernelGGL(kern, dim3((unsigned)nh), dim3(256), 0, stream, q, k, v, g, beta, p.S, o,
                         p.accept, p.H, p.m, nh);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_multi_kernel<DK, DV, TIn, TOut>), dim3((unsigned)nh), dim3(256), 0,
                     stream, q, k, v, g, beta, p.S, o, p.accept, p.H, p.m, nh);
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
