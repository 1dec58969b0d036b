// Matrix-core chunked KDA forward for gfx950: bf16 activations, dk = dv = 128, chunk 64.
//
// The chunked algebra (from the recurrence S_r = (I - b_r k_r k_r^T) D_r S_{r-1} + b_r k_r v_r^T)
// for a 64-token chunk entered with state S, G_r = sum_{j<=r} g_j per key channel:
//   U' = M (V - Kbar S),  M = (I + A)^{-1} diag(b),  A[r][j] = b_r sum_c k_r k_j e^{G_r - G_j} (j < r)
//   O  = Qbar S + Aqk U', Aqk[r][j] = sum_c q_r k_j e^{G_r - G_j} (j <= r)
//   S <- Diag(e^{G_C}) S + Ktil^T U',  Kbar = K e^{G}, Qbar = Q e^{G}, Ktil = K e^{G_C - G}.
//
// Two kernels.
//  prep_kernel (one workgroup per chunk and head, all chunks in parallel): the per-channel
//    cumulative log-decay; A and Aqk on the matrix cores; the inverse (I + A)^{-1} by
//    blocked forward substitution in LDS; and every operand the recurrence needs, stored
//    in the workspace already in MFMA lane order ("fragments", 1 KiB = 64 lanes x 8 fp16)
//    so that each later load is one coalesced 16-byte load per lane.
//    A and Aqk are built from 16-token tiles whose exponent is measured from the state before
//    the row tile: the row factor e^{G_r - ref} lies in [e^-80, 1] and the column factor
//    e^{ref - G_j} is <= 1 off the diagonal and in [1, e^80] on it, because each step's
//    log-decay is >= -5 (orkas.ai Kimi K3 page, "Eine Untergrenze, die einen GPU-Codepfad
//    beseitigte"). The diagonal tiles therefore run the same dense MFMA as the others; their
//    operands need bf16's exponent range (fp16 would overflow at e^80), and are split into
//    bf16 hi + lo pairs (three products) to keep 16 bits of precision. Off-diagonal factors
//    are <= 1 and use fp16 (11-bit significand) directly.
//  rec_kernel (one workgroup per sequence, head and 16 value columns, serial over chunks):
//    the fp32 state slice S[128][16] lives in MFMA accumulators for the whole sequence;
//    four waves split the 128 key rows. Per chunk: the state strip is all-gathered in
//    fp16 through LDS, each wave forms complete Kbar S and Qbar S for its own 16 chunk rows,
//    Y = V - Kbar S is all-gathered, U' = M Y, then the outputs Qbar S + Aqk U' (Aqk and U'
//    split into fp16 hi + lo) and the wave's rows of the state update. Columns of S evolve independently
//    (the transition acts on the key side only), so splitting the value columns over
//    workgroups is exact and needs no communication.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = 64;
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int NSTRIP = DV / 16;  // 16-column strips per (sequence, head)

// Workspace block of one (chunk, head), byte offsets. Fragment f of a group starts at
// group + f * 1024; lane l's eight fp16 values at + l * 16.
constexpr int OFF_KB = 0;        // -Kbar as A operand: [k-step over dk (4)][row tile (4)]
constexpr int OFF_QB = 16384;    // Qbar, same order
constexpr int OFF_KT = 32768;    // Ktil^T: [dk tile (8)][k-step over chunk rows (2)]
constexpr int OFF_M = 49152;     // M: [row tile (4)][k-step (2)]
constexpr int OFF_AHI = 57344;   // Aqk hi: [row tile (4)][k-step (2)]
constexpr int OFF_ALO = 65536;   // Aqk lo
constexpr int OFF_GAM = 73728;   // e^{G_C}, fp32 [128]
constexpr size_t kBlockBytes = 74240;

struct SeqInfo {
  int64_t tok0;  // first token of the sequence in the packed T axis
  int64_t len;
  int64_t cid0;  // first chunk of the sequence in the workspace
};

__device__ __forceinline__ SeqInfo seq_info(int n, const int32_t* cu, const int32_t* chunk_off,
                                            int T) {
  SeqInfo s;
  if (cu) {
    const int64_t a = min(max((int64_t)cu[n], (int64_t)0), (int64_t)T);
    const int64_t e = min(max((int64_t)cu[n + 1], a), (int64_t)T);
    s.tok0 = a;
    s.len = e - a;
    s.cid0 = chunk_off[n];
  } else {
    s.tok0 = (int64_t)n * T;
    s.len = T;
    s.cid0 = (int64_t)n * ((T + C - 1) / C);
  }
  return s;
}

// chunk_off[n] = number of chunks of sequences 0..n-1 (lengths clamped as in seq_info).
__global__ __launch_bounds__(256) void plan_kernel(const int32_t* __restrict__ cu, int n_seq,
                                                   int T, int32_t* __restrict__ chunk_off) {
  __shared__ int64_t part[256];
  const int t = threadIdx.x;
  const int per = (n_seq + 255) / 256;
  const int lo = min(t * per, n_seq), hi = min(lo + per, n_seq);
  int64_t sum = 0;
  for (int n = lo; n < hi; ++n) {
    const int64_t a = min(max((int64_t)cu[n], (int64_t)0), (int64_t)T);
    const int64_t e = min(max((int64_t)cu[n + 1], a), (int64_t)T);
    sum += (e - a + C - 1) / C;
  }
  part[t] = sum;
  __syncthreads();
  if (t == 0) {
    int64_t acc = 0;
    for (int i = 0; i < 256; ++i) {
      const int64_t x = part[i];
      part[i] = acc;
      acc += x;
    }
  }
  __syncthreads();
  int64_t acc = part[t];
  for (int n = lo; n < hi; ++n) {
    chunk_off[n] = (int32_t)acc;
    const int64_t a = min(max((int64_t)cu[n], (int64_t)0), (int64_t)T);
    const int64_t e = min(max((int64_t)cu[n + 1], a), (int64_t)T);
    acc += (e - a + C - 1) / C;
  }
  if (t == 255) chunk_off[n_seq] = (int32_t)acc;
}

// ---------------------------------------------------------------- prep
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// One workgroup per (chunk, head); wave a owns row tile a (chunk rows 16a .. 16a+15). In the
// MFMA fragment layout lane l of wave a holds row 16a + (l & 15) and, for each of the four
// 32-channel k-steps, the eight channels 32 ks + kslot(l >> 4, i). Every per-element quantity
// is formed once, in registers, in that layout:
//   rf = e^{G_r - ref_a}   (ref_a = G at the last token before tile a)   in [e^-80, 1]
//   cf = e^{Gend_a - G_r}  (Gend_a = G at the last token of tile a)       in [e^-80, 1]
// The row operand of tile a is k rf (q rf), its diagonal column operand k / rf (in [1, e^80]
// times k, bf16 range), and the column operand it lends to later tiles b > a is k cf, scaled
// there by the per-channel factor e^{ref_b - Gend_a} <= 1. Kbar, Qbar and Ktil follow from the
// same values times per-channel constants.
__global__ __launch_bounds__(256, 2) void prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ beta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off, int T, int H,
    int n_seq, uint8_t* __restrict__ ws) {
  constexpr int GSR = DK + 4;   // log2 cumulative decay rows (fp32)
  constexpr int KTR = C + 8;    // Ktil^T rows (fp16, channel-major)
  // R1: G (fp32 [64][GSR]) -> Ktil^T (fp16 [128][KTR]) -> A, Aqk (fp32 [64][64] each)
  // R2: column operands k cf (fp32, fragment order [tile][ks][lane][8]) -> T (fp32 [64][64]), X
  __shared__ __align__(16) float R1[64 * GSR];
  __shared__ __align__(16) float R2[4 * 4 * 64 * 8];
  __shared__ __align__(16) float REF2[4][DK], END2[4][DK], PCH[4][DK], ECH[4][DK], XCH[3][DK];
  __shared__ float Bs[C];
  float* Gs = R1;
  _Float16* KtT = reinterpret_cast<_Float16*>(R1);
  float* A32 = R1;
  float* AQ32 = R1 + 64 * 64;
  float* T32 = R2;
  float* Xs = R2 + 64 * 64;

  const int h = blockIdx.x % H;
  const int64_t cid = blockIdx.x / H;
  int n;
  int64_t c_in;
  if (cu) {
    if (cid >= chunk_off[n_seq]) return;
    int lo = 0, hi = n_seq - 1;  // last n with chunk_off[n] <= cid
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (chunk_off[mid] <= cid) lo = mid; else hi = mid - 1;
    }
    n = lo;
    c_in = cid - chunk_off[n];
  } else {
    const int64_t ncs = (T + C - 1) / C;
    n = (int)(cid / ncs);
    c_in = cid % ncs;
    if (n >= n_seq) return;
  }
  const SeqInfo si = seq_info(n, cu, chunk_off, T);
  const int64_t tok0 = si.tok0 + c_in * C;
  const int Cn = (int)min((int64_t)C, si.len - c_in * C);
  uint8_t* blk = ws + ((size_t)cid * H + h) * kBlockBytes;

  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l = t & 63, gq = l >> 4, m = l & 15;

  // this lane's k and q elements (row 16w + m, fragment channels), issued first so their
  // latency overlaps phase 1
  const int row = 16 * w + m;
  const bool row_ok = row < Cn;
  u16x4 kraw[4][2], qraw[4][2];
  {
    const int64_t erow = ((tok0 + min(row, Cn - 1)) * H + h) * DK;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c0 = 32 * ks + 4 * gq;
      kraw[ks][0] = *reinterpret_cast<const u16x4*>(k + erow + c0);
      kraw[ks][1] = *reinterpret_cast<const u16x4*>(k + erow + c0 + 16);
      qraw[ks][0] = *reinterpret_cast<const u16x4*>(q + erow + c0);
      qraw[ks][1] = *reinterpret_cast<const u16x4*>(q + erow + c0 + 16);
    }
  }
  // ---- phase 1: g rows into LDS (rows past the end read as 0), beta
  {
    const int r = t >> 2, cb = t & 3;
    const bool ok = r < Cn;
    const int64_t e = ((tok0 + min(r, Cn - 1)) * H + h) * DK + cb * 32;
    u16x8 gv[4];
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) gv[vv] = *reinterpret_cast<const u16x8*>(g + e + 8 * vv);
    const uint16_t braw = beta[(tok0 + min(t & (C - 1), Cn - 1)) * H + h];
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) {
      floatx4 lo4, hi4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo4[i] = ok ? bf16_bits_to_f32(gv[vv][i]) : 0.f;
        hi4[i] = ok ? bf16_bits_to_f32(gv[vv][i + 4]) : 0.f;
      }
      *reinterpret_cast<floatx4*>(&Gs[r * GSR + cb * 32 + 8 * vv]) = lo4;
      *reinterpret_cast<floatx4*>(&Gs[r * GSR + cb * 32 + 8 * vv + 4]) = hi4;
    }
    if (t < C) Bs[t] = (t < Cn) ? bf16_bits_to_f32(braw) : 0.f;
  }
  __syncthreads();
  // ---- cumulative log-decay per channel (log2 units) and the per-channel constants
  if (t < DK) {
    float col[C];
#pragma unroll
    for (int r = 0; r < C; ++r) col[r] = Gs[r * GSR + t];
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      acc += col[r];
      col[r] = acc * kLog2e;
      Gs[r * GSR + t] = col[r];
    }
    float ref[4], end[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      ref[a] = a ? col[16 * a - 1] : 0.f;
      end[a] = col[16 * a + 15];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      REF2[a][t] = ref[a];
      END2[a][t] = end[a];
      PCH[a][t] = exp2f(ref[a]);             // e^{ref_a}: Kbar = (k rf) e^{ref_a}
      ECH[a][t] = exp2f(end[3] - end[a]);    // e^{G_C - Gend_a}: Ktil = (k cf) e^{G_C - Gend_a}
    }
    XCH[0][t] = exp2f(end[1] - end[0]);      // column factor of block (2, 0)
    XCH[1][t] = exp2f(end[2] - end[0]);      // (3, 0)
    XCH[2][t] = exp2f(end[2] - end[1]);      // (3, 1)
    reinterpret_cast<float*>(blk + OFF_GAM)[t] = exp2f(end[3]);
  }
  __syncthreads();
  // ---- phase 2: this lane's 32 elements of row 16w + m (k, q loaded before phase 1)
  float kr[4][8], qr[4][8], kd[4][8];  // k rf, q rf, k / rf
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int c0 = 32 * ks + 4 * gq;
    const u16x4 k0 = kraw[ks][0], k1 = kraw[ks][1], q0 = qraw[ks][0], q1 = qraw[ks][1];
    const floatx4 g0 = *reinterpret_cast<const floatx4*>(&Gs[row * GSR + c0]);
    const floatx4 g1 = *reinterpret_cast<const floatx4*>(&Gs[row * GSR + c0 + 16]);
    const floatx4 r0 = *reinterpret_cast<const floatx4*>(&REF2[w][c0]);
    const floatx4 r1 = *reinterpret_cast<const floatx4*>(&REF2[w][c0 + 16]);
    const floatx4 e0 = *reinterpret_cast<const floatx4*>(&END2[w][c0]);
    const floatx4 e1 = *reinterpret_cast<const floatx4*>(&END2[w][c0 + 16]);
    const floatx4 p0 = *reinterpret_cast<const floatx4*>(&PCH[w][c0]);
    const floatx4 p1 = *reinterpret_cast<const floatx4*>(&PCH[w][c0 + 16]);
    half8 knf, qbf;
    floatx4 kc0, kc1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = i & 3;
      const float kv = row_ok ? bf16_bits_to_f32(i < 4 ? k0[j] : k1[j]) : 0.f;
      const float qv = row_ok ? bf16_bits_to_f32(i < 4 ? q0[j] : q1[j]) : 0.f;
      const float gg = i < 4 ? g0[j] : g1[j];
      const float rf = exp2f(gg - (i < 4 ? r0[j] : r1[j]));
      const float cf = exp2f((i < 4 ? e0[j] : e1[j]) - gg);
      kr[ks][i] = kv * rf;
      qr[ks][i] = qv * rf;
      kd[ks][i] = kv * __builtin_amdgcn_rcpf(rf);
      const float kcv = kv * cf;
      if (i < 4) kc0[j] = kcv; else kc1[j] = kcv;
      const float pe = i < 4 ? p0[j] : p1[j];
      knf[i] = static_cast<_Float16>(-kr[ks][i] * pe);
      qbf[i] = static_cast<_Float16>(qr[ks][i] * pe);
    }
    // Kbar (negated) and Qbar fragments [ks][row tile w]
    *reinterpret_cast<half8*>(blk + OFF_KB + (ks * 4 + w) * 1024 + l * 16) = knf;
    *reinterpret_cast<half8*>(blk + OFF_QB + (ks * 4 + w) * 1024 + l * 16) = qbf;
    // column operand k cf lent to later row tiles
    float* kcp = R2 + ((w * 4 + ks) * 64 + l) * 8;
    *reinterpret_cast<floatx4*>(kcp) = kc0;
    *reinterpret_cast<floatx4*>(kcp + 4) = kc1;
  }
  __syncthreads();  // every wave has read G: R1 is reused for Ktil^T
  // Ktil = (k cf) e^{G_C - Gend_w}, transposed to channel-major for its fragments
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const float* kcp = R2 + ((w * 4 + ks) * 64 + l) * 8;
    const int c0 = 32 * ks + 4 * gq;
    const floatx4 v0 = *reinterpret_cast<const floatx4*>(kcp);
    const floatx4 v1 = *reinterpret_cast<const floatx4*>(kcp + 4);
    const floatx4 x0 = *reinterpret_cast<const floatx4*>(&ECH[w][c0]);
    const floatx4 x1 = *reinterpret_cast<const floatx4*>(&ECH[w][c0 + 16]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      KtT[(c0 + i) * KTR + row] = static_cast<_Float16>(v0[i] * x0[i]);
      KtT[(c0 + 16 + i) * KTR + row] = static_cast<_Float16>(v1[i] * x1[i]);
    }
  }
  __syncthreads();
  // ---- Ktil^T fragments [dk tile][ks over chunk rows]: four per wave
#pragma unroll
  for (int jf = 0; jf < 4; ++jf) {
    const int f = w * 4 + jf;
    const int mt = f >> 1, ks = f & 1;
    const _Float16* src = KtT + (16 * mt + m) * KTR + 32 * ks + 4 * gq;
    const half4 a0 = *reinterpret_cast<const half4*>(src);
    const half4 a1 = *reinterpret_cast<const half4*>(src + 16);
    half8 kt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kt[i] = a0[i];
      kt[i + 4] = a1[i];
    }
    *reinterpret_cast<half8*>(blk + OFF_KT + f * 1024 + l * 16) = kt;
  }
  // ---- A = beta K K^T and Aqk = Q K^T tiles of row tile w on the matrix cores
  floatx4 akk[4], aqk[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) akk[bb] = aqk[bb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    half8 rk16, rq16;
    bf16x8 rkh, rkl, rqh, rql, ch, cl;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      rk16[i] = static_cast<_Float16>(kr[ks][i]);
      rq16[i] = static_cast<_Float16>(qr[ks][i]);
      __bf16 hh, ll;
      split_bf16(kr[ks][i], hh, ll); rkh[i] = hh; rkl[i] = ll;
      split_bf16(qr[ks][i], hh, ll); rqh[i] = hh; rql[i] = ll;
      split_bf16(kd[ks][i], hh, ll); ch[i] = hh; cl[i] = ll;
    }
    // diagonal tile: column factor up to e^80, split bf16
    akk[w] = mfma_bf16(rkh, ch, akk[w]);
    akk[w] = mfma_bf16(rkh, cl, akk[w]);
    akk[w] = mfma_bf16(rkl, ch, akk[w]);
    aqk[w] = mfma_bf16(rqh, ch, aqk[w]);
    aqk[w] = mfma_bf16(rqh, cl, aqk[w]);
    aqk[w] = mfma_bf16(rql, ch, aqk[w]);
    // earlier tiles: factors <= 1, fp16
#pragma unroll
    for (int bb = 0; bb < 3; ++bb) {
      if (bb >= w) break;
      const float* kcp = R2 + ((bb * 4 + ks) * 64 + l) * 8;
      const floatx4 c0 = *reinterpret_cast<const floatx4*>(kcp);
      const floatx4 c1 = *reinterpret_cast<const floatx4*>(kcp + 4);
      floatx4 x0 = {1.f, 1.f, 1.f, 1.f}, x1 = x0;
      if (bb < w - 1) {  // blocks (2,0), (3,0), (3,1): e^{ref_w - Gend_bb}
        const int xi = (w == 2) ? 0 : (bb == 0 ? 1 : 2);
        x0 = *reinterpret_cast<const floatx4*>(&XCH[xi][32 * ks + 4 * gq]);
        x1 = *reinterpret_cast<const floatx4*>(&XCH[xi][32 * ks + 16 + 4 * gq]);
      }
      half8 c16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c16[i] = static_cast<_Float16>(c0[i] * x0[i]);
        c16[i + 4] = static_cast<_Float16>(c1[i] * x1[i]);
      }
      akk[bb] = mfma_f16(rk16, c16, akk[bb]);
      aqk[bb] = mfma_f16(rq16, c16, aqk[bb]);
    }
  }
  __syncthreads();  // Ktil^T and the lent column operands are dead: R1, R2 reused
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * gq + i, jc = 16 * bb + m;
      A32[r * 64 + jc] = (bb <= w && jc < r) ? Bs[r] * akk[bb][i] : 0.f;
      AQ32[r * 64 + jc] = (bb <= w && jc <= r) ? aqk[bb][i] : 0.f;
    }
  }
  for (int i = t; i < 64 * 64; i += 256) T32[i] = 0.f;
  __syncthreads();
  // ---- T = (I + A)^{-1}: diagonal 16x16 blocks by substitution (wave w, lane = column)
  if (l < 16) {
    const int j = l, o = 16 * w;
    float col[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float sacc = 0.f;
#pragma unroll
      for (int mm = 0; mm < i; ++mm)
        if (mm >= j) sacc += A32[(o + i) * 64 + o + mm] * col[mm];
      col[i] = (i < j) ? 0.f : (i == j ? 1.f : -sacc);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) T32[(o + i) * 64 + o + j] = col[i];
  }
  __syncthreads();
  // ---- off-diagonal blocks, by distance from the diagonal:
  //      T_ab = -T_aa * sum_{c=b}^{a-1} A_ac T_cb
  {
    const int i = t >> 4, jj = t & 15;
#pragma unroll
    for (int L = 1; L < 4; ++L) {
      for (int a = L; a < 4; ++a) {
        const int bb = a - L;
        float x = 0.f;
        for (int cc = bb; cc < a; ++cc)
#pragma unroll
          for (int mm = 0; mm < 16; ++mm)
            x += A32[(16 * a + i) * 64 + 16 * cc + mm] * T32[(16 * cc + mm) * 64 + 16 * bb + jj];
        Xs[(a - L) * 256 + i * 16 + jj] = x;
      }
      __syncthreads();
      for (int a = L; a < 4; ++a) {
        const int bb = a - L;
        float x = 0.f;
#pragma unroll
        for (int mm = 0; mm < 16; ++mm)
          x += T32[(16 * a + i) * 64 + 16 * a + mm] * Xs[(a - L) * 256 + mm * 16 + jj];
        T32[(16 * a + i) * 64 + 16 * bb + jj] = -x;
      }
      __syncthreads();
    }
  }
  // ---- M = T diag(beta) and Aqk hi/lo fragments: [row tile][ks]
#pragma unroll
  for (int jf = 0; jf < 2; ++jf) {
    const int f = (t >> 6) + 4 * jf;  // 0..7
    const int mt = f >> 1, ks = f & 1;
    const int rr = 16 * mt + m;
    half8 mf, ah, al;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int cc = 32 * ks + kslot(gq, i);
      mf[i] = static_cast<_Float16>(T32[rr * 64 + cc] * Bs[cc]);
      _Float16 hh, ll;
      split_f16(AQ32[rr * 64 + cc], hh, ll);
      ah[i] = hh;
      al[i] = ll;
    }
    *reinterpret_cast<half8*>(blk + OFF_M + f * 1024 + l * 16) = mf;
    *reinterpret_cast<half8*>(blk + OFF_AHI + f * 1024 + l * 16) = ah;
    *reinterpret_cast<half8*>(blk + OFF_ALO + f * 1024 + l * 16) = al;
  }
}

// ---------------------------------------------------------------- rec
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes): loads past the end return zero and stores
// past the end are dropped, which is how partial chunks are masked without branches.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = (int)min(max(bytes, (int64_t)0), (int64_t)0x7fffffff);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ half8 ld_frag(rsrc_t r, int lane_off, int off) {
  return __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, off, 0));
}

template <typename TOut, int NT>
__global__ __launch_bounds__(256) void rec_kernel(
    const uint16_t* __restrict__ v, const float* __restrict__ S0, TOut* __restrict__ o,
    float* __restrict__ S_T, const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off,
    int T, int H, int n_seq, int64_t max_chunks, const uint8_t* __restrict__ ws) {
  // A workgroup owns NT strips of 16 value columns; every operand fragment a wave loads
  // feeds NT matrix products. Two fp16 exchanges per chunk, double-buffered: the state
  // strips (all 128 key rows), so every wave can form complete Kbar S and Qbar S for its own
  // 16 chunk rows, and Y = V - Kbar S (all 64 chunk rows) for U' = M Y. Both are stored
  // column-major ([column][row]) so the rows a lane needs for a B operand are contiguous,
  // with rows padded by 8 halves against bank conflicts.
  constexpr int NG = NSTRIP / NT;  // strip groups per (sequence, head)
  constexpr int SR = DK + 8, YR = C + 8;
  __shared__ __align__(16) _Float16 sx[2][NT * 16][SR];
  __shared__ __align__(16) _Float16 yx[2][NT * 16][YR];

  // XCD-aware placement: the strip groups of one (sequence, head) share an XCD and its L2.
  const int b = blockIdx.x;
  const int xcd = b & 7, rest = b >> 3;
  const int sg = rest % NG;
  const int64_t pair = (int64_t)(rest / NG) * 8 + xcd;
  if (pair >= (int64_t)n_seq * H) return;
  const int n = (int)(pair / H), h = (int)(pair % H);
  const SeqInfo si = seq_info(n, cu, chunk_off, T);
  // a malformed cu_seqlens cannot make the chunk walk leave the workspace
  const int64_t nc = max((int64_t)0, min((si.len + C - 1) / C, max_chunks - si.cid0));

  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l = t & 63, gq = l >> 4, nn = l & 15;
  const int64_t s_base = pair * DK * DV;
  const int row_stride = H * DV;  // elements between consecutive tokens
  int col[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) col[nt] = 16 * (NT * sg + nt) + nn;

  // this wave's state rows 32w + 16u + 4gq + i (u = 0, 1), columns col[nt]
  floatx4 s[NT][2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s[nt][u][i] = S0 ? S0[s_base + (int64_t)(32 * w + 16 * u + 4 * gq + i) * DV + col[nt]] : 0.f;

  // per-lane byte offsets, fixed for the whole sequence
  const int frag_off = l * 16;
  int v_off[NT][4], o_off[NT][4];  // this wave's chunk rows 16w + 4gq + i
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v_off[nt][i] = ((16 * w + 4 * gq + i) * row_stride + col[nt]) * 2;
      o_off[nt][i] = ((16 * w + 4 * gq + i) * row_stride + col[nt]) * (int)sizeof(TOut);
    }
  const int gam_off = OFF_GAM + (32 * w + 4 * gq) * 4;

  const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
  half8 kn[4], qb[4], mf[4][2], ahi[2], alo[2], kt[2][2];
  floatx4 gam[2], gam_nx[2];  // e^{G_C} of the current and of the next chunk
  uint16_t vraw[NT][4];

  // buffer bases advance by a fixed stride per chunk
  const uint8_t* blk_base = ws + ((size_t)si.cid0 * H + h) * kBlockBytes;
  const size_t blk_step = (size_t)H * kBlockBytes;
  const uint16_t* v_base = v + (si.tok0 * H + h) * DV;
  TOut* o_base = o + (si.tok0 * H + h) * DV;
  const size_t tok_step = (size_t)C * row_stride;
  // bytes of the chunk's rows of this head, up to the end of its last valid row
  auto rows_bytes = [&](int64_t c, int elem) -> int64_t {
    const int64_t rows = min((int64_t)C, si.len - c * C);
    return ((rows - 1) * row_stride + DV) * elem;
  };

  auto load_kq = [&](rsrc_t r) {  // this wave's row tile, all four dk k-steps; e^{G_C}
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kn[j] = ld_frag(r, frag_off, OFF_KB + (j * 4 + w) * 1024);
      qb[j] = ld_frag(r, frag_off, OFF_QB + (j * 4 + w) * 1024);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
      gam_nx[u] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, gam_off, 64 * u, 0));
  };
  auto load_m = [&](rsrc_t r) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) mf[mt][ks] = ld_frag(r, frag_off, OFF_M + (mt * 2 + ks) * 1024);
  };
  auto load_a = [&](rsrc_t r) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      ahi[ks] = ld_frag(r, frag_off, OFF_AHI + (w * 2 + ks) * 1024);
      alo[ks] = ld_frag(r, frag_off, OFF_ALO + (w * 2 + ks) * 1024);
    }
  };
  auto load_kt = [&](rsrc_t r) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) kt[u][ks] = ld_frag(r, frag_off, OFF_KT + ((2 * w + u) * 2 + ks) * 1024);
  };
  auto load_v = [&](int64_t c) {
    const rsrc_t r = make_rsrc(v_base + c * tok_step, rows_bytes(c, 2));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) vraw[nt][i] = __builtin_amdgcn_raw_buffer_load_b16(r, v_off[nt][i], 0, 0);
  };

  if (nc > 0) {  // same issue order as in the loop, so the loop's memory waits stay partial
    const rsrc_t r0 = make_rsrc(blk_base, (int64_t)kBlockBytes);
    load_kq(r0);
    load_v(0);
    load_m(r0);
    load_a(r0);
    load_kt(r0);
  }
  int buf = 0;
  for (int64_t c = 0; c < nc; ++c) {
    // operands of the next chunk are loaded right after their use in this one (the last
    // chunk reloads itself), unconditionally and in a fixed order, so every load has a
    // chunk's time to land and the loop carries no branch
    const int64_t cn = min(c + 1, nc - 1);
    const rsrc_t rn = make_rsrc(blk_base + cn * blk_step, (int64_t)kBlockBytes);
    gam[0] = gam_nx[0];
    gam[1] = gam_nx[1];
    // -- all-gather the state strips in fp16
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        half4 hv;
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = static_cast<_Float16>(s[nt][u][i]);
        *reinterpret_cast<half4*>(&sx[buf][16 * nt + nn][32 * w + 16 * u + 4 * gq]) = hv;
      }
    __syncthreads();
    // -- complete -Kbar S and Qbar S for this wave's 16 chunk rows
    floatx4 X[NT], QS[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) X[nt] = QS[nt] = zero;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        half8 bs;
        const _Float16* sp = &sx[buf][16 * nt + nn][32 * j + 4 * gq];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bs[i] = sp[i];
          bs[i + 4] = sp[16 + i];
        }
        X[nt] = mfma_f16(kn[j], bs, X[nt]);
        QS[nt] = mfma_f16(qb[j], bs, QS[nt]);
      }
    }
    load_kq(rn);
    // -- Y = V - Kbar S for this wave's rows, all-gathered in fp16
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      half4 hy;
#pragma unroll
      for (int i = 0; i < 4; ++i) hy[i] = static_cast<_Float16>(X[nt][i] + bf16_bits_to_f32(vraw[nt][i]));
      *reinterpret_cast<half4*>(&yx[buf][16 * nt + nn][16 * w + 4 * gq]) = hy;
    }
    load_v(cn);
    __syncthreads();
    // -- U' = M Y, all 64 rows (each wave keeps a full copy), split into fp16 hi + lo
    half8 uh[NT][2], ul[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      half8 by[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const _Float16* yp = &yx[buf][16 * nt + nn][32 * ks + 4 * gq];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          by[ks][i] = yp[i];
          by[ks][i + 4] = yp[16 + i];
        }
      }
      floatx4 U[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        U[mt] = mfma_f16(mf[mt][0], by[0], zero);
        U[mt] = mfma_f16(mf[mt][1], by[1], U[mt]);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          _Float16 hh, ll;
          split_f16(i < 4 ? U[2 * ks][i] : U[2 * ks + 1][i - 4], hh, ll);
          uh[nt][ks][i] = hh;
          ul[nt][ks][i] = ll;
        }
    }
    load_m(rn);
    // -- outputs of this wave's rows: Qbar S + Aqk U' (for rows < 32 the second k-step
    //    multiplies the zero upper part of Aqk; it is kept so the loop body has no branch)
    {
      const rsrc_t ro = make_rsrc(o_base + c * tok_step, rows_bytes(c, (int)sizeof(TOut)));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        floatx4 acc = QS[nt];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          acc = mfma_f16(ahi[ks], uh[nt][ks], acc);
          acc = mfma_f16(ahi[ks], ul[nt][ks], acc);
          acc = mfma_f16(alo[ks], uh[nt][ks], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (sizeof(TOut) == 4)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i]), ro, o_off[nt][i], 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(acc[i]), ro, o_off[nt][i], 0, 0);
        }
      }
    }
    load_a(rn);
    // -- this wave's state rows: S = Diag(e^{G_C}) S + Ktil^T U'
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        s[nt][u] *= gam[u];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          s[nt][u] = mfma_f16(kt[u][ks], uh[nt][ks], s[nt][u]);
          s[nt][u] = mfma_f16(kt[u][ks], ul[nt][ks], s[nt][u]);
        }
      }
    load_kt(rn);
    buf ^= 1;
  }
  if (S_T) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S_T[s_base + (int64_t)(32 * w + 16 * u + 4 * gq + i) * DV + col[nt]] = s[nt][u][i];
  }
}

int64_t max_chunks(const ChunkPlan& p) {
  const int64_t per = (p.T + C - 1) / C;
  return p.cu_seqlens ? per + p.n_seq : (int64_t)p.B * per;
}

size_t chunk_table_offset(const ChunkPlan& p) {
  return (size_t)max_chunks(p) * p.H * kBlockBytes;
}

}  // namespace

bool fast_path_applies(const ChunkPlan& p) {
  return p.act_bf16 && p.dk == DK && p.dv == DV && p.chunk == C;
}

size_t fast_workspace_bytes(const ChunkPlan& p) {
  size_t bytes = chunk_table_offset(p);
  if (p.cu_seqlens) bytes += ((sizeof(int32_t) * (p.n_seq + 1) + 255) / 256) * 256;
  return bytes;
}

hipError_t launch_chunk_fast(const ChunkPlan& p, hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(p.workspace);
  int32_t* chunk_off = nullptr;
  if (p.cu_seqlens) {
    chunk_off = reinterpret_cast<int32_t*>(ws + chunk_table_offset(p));
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, p.cu_seqlens, p.n_seq, p.T,
                       chunk_off);
  }
  const int64_t prep_blocks = max_chunks(p) * p.H;
  if (prep_blocks > 0)
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)prep_blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k),
                       static_cast<const uint16_t*>(p.g), static_cast<const uint16_t*>(p.beta),
                       p.cu_seqlens, chunk_off, p.T, p.H, p.n_seq, ws);
  const int64_t pairs = (int64_t)p.n_seq * p.H;
  // Few (sequence, head) pairs: the chunk walk is latency bound, so one 16-column strip per
  // workgroup maximises parallelism. Many pairs (at least four strip workgroups per CU): two
  // strips per workgroup halve the operand traffic per column.
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  const bool two = pairs * NSTRIP >= 4LL * n_cu;
  const int64_t rec_blocks = ((pairs + 7) / 8) * 8 * (two ? NSTRIP / 2 : NSTRIP);
  const dim3 grid((unsigned)rec_blocks), block(256);
  const uint16_t* vv = static_cast<const uint16_t*>(p.v);
  const int64_t mc = max_chunks(p);
  if (p.out_bf16) {
    uint16_t* oo = static_cast<uint16_t*>(p.o);
    if (two)
      hipLaunchKernelGGL((rec_kernel<uint16_t, 2>), grid, block, 0, stream, vv, p.S0, oo, p.S_T,
                         p.cu_seqlens, chunk_off, p.T, p.H, p.n_seq, mc, ws);
    else
      hipLaunchKernelGGL((rec_kernel<uint16_t, 1>), grid, block, 0, stream, vv, p.S0, oo, p.S_T,
                         p.cu_seqlens, chunk_off, p.T, p.H, p.n_seq, mc, ws);
  } else {
    float* oo = static_cast<float*>(p.o);
    if (two)
      hipLaunchKernelGGL((rec_kernel<float, 2>), grid, block, 0, stream, vv, p.S0, oo, p.S_T,
                         p.cu_seqlens, chunk_off, p.T, p.H, p.n_seq, mc, ws);
    else
      hipLaunchKernelGGL((rec_kernel<float, 1>), grid, block, 0, stream, vv, p.S0, oo, p.S_T,
                         p.cu_seqlens, chunk_off, p.T, p.H, p.n_seq, mc, ws);
  }
  return hipGetLastError();
}

}  // namespace kda
