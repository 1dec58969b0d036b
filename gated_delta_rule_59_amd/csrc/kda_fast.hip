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

// LDS row strides (elements), padded against bank conflicts.
constexpr int GS = DK + 1;  // fp32 cumulative log2-decay rows
constexpr int KS = DK + 2;  // bf16 k and q rows

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

__device__ __forceinline__ float bfv(const uint16_t* p) { return bf16_bits_to_f32(*p); }

// ---------------------------------------------------------------- prep: A and Aqk tiles
// Wave `a` computes row tile a of A and Aqk: blocks (a, b) for b <= a, K = 128 in four
// k-steps of 32 channels.
template <int A_TILE>
__device__ __forceinline__ void tile_products(const uint16_t* Ks, const uint16_t* Qs,
                                              const float* Gs, int l, floatx4 (&akk)[4],
                                              floatx4 (&aqk)[4]) {
  const int g = l >> 4, m = l & 15;
  const int rr = 16 * A_TILE + m;          // row operand: chunk row
  const float* ref = Gs + (A_TILE > 0 ? 16 * A_TILE - 1 : 0) * GS;  // log2-decay before the row tile
#pragma unroll
  for (int b = 0; b < 4; ++b) akk[b] = aqk[b] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    float rk[8], rq[8], refc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = 32 * ks + kslot(g, i);
      refc[i] = A_TILE > 0 ? ref[c] : 0.f;
      const float f = exp2f(Gs[rr * GS + c] - refc[i]);
      rk[i] = bfv(Ks + rr * KS + c) * f;
      rq[i] = bfv(Qs + rr * KS + c) * f;
    }
    half8 rk16, rq16;
    bf16x8 rkh, rkl, rqh, rql;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      rk16[i] = static_cast<_Float16>(rk[i]);
      rq16[i] = static_cast<_Float16>(rq[i]);
      __bf16 h, lo;
      split_bf16(rk[i], h, lo); rkh[i] = h; rkl[i] = lo;
      split_bf16(rq[i], h, lo); rqh[i] = h; rql[i] = lo;
    }
#pragma unroll
    for (int b = 0; b <= A_TILE; ++b) {
      const int jj = 16 * b + m;  // column operand: chunk row j
      float cv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = 32 * ks + kslot(g, i);
        cv[i] = bfv(Ks + jj * KS + c) * exp2f(refc[i] - Gs[jj * GS + c]);
      }
      if (b < A_TILE) {  // factors <= 1: fp16
        half8 c16;
#pragma unroll
        for (int i = 0; i < 8; ++i) c16[i] = static_cast<_Float16>(cv[i]);
        akk[b] = mfma_f16(rk16, c16, akk[b]);
        aqk[b] = mfma_f16(rq16, c16, aqk[b]);
      } else {  // diagonal tile: column factor up to e^80, bf16 hi + lo
        bf16x8 ch, cl;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __bf16 h, lo;
          split_bf16(cv[i], h, lo);
          ch[i] = h;
          cl[i] = lo;
        }
        akk[b] = mfma_bf16(rkh, ch, akk[b]);
        akk[b] = mfma_bf16(rkh, cl, akk[b]);
        akk[b] = mfma_bf16(rkl, ch, akk[b]);
        aqk[b] = mfma_bf16(rqh, ch, aqk[b]);
        aqk[b] = mfma_bf16(rqh, cl, aqk[b]);
        aqk[b] = mfma_bf16(rql, ch, aqk[b]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ beta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off, int T, int H,
    int n_seq, uint8_t* __restrict__ ws) {
  // Phase 1 layout: Ks, Qs (bf16 [64][KS]) then Gs (fp32 [64][GS]).
  // Phase 2 (after the products): A32, AQ32 over Ks/Qs; T32, Xs over Gs.
  __shared__ __align__(16) unsigned char smem[2 * 64 * KS * 2 + 64 * GS * 4];
  __shared__ float Bs[C];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Qs = Ks + 64 * KS;
  float* Gs = reinterpret_cast<float*>(smem + 2 * 64 * KS * 2);
  float* A32 = reinterpret_cast<float*>(smem);  // [64][64]
  float* AQ32 = A32 + 64 * 64;                  // [64][64]
  float* T32 = Gs;                              // [64][64]
  float* Xs = Gs + 64 * 64;                     // [3][16][16]

  const int h = blockIdx.x % H;
  const int64_t cid = blockIdx.x / H;
  // locate the chunk: sequence n and chunk index within it
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
  // ---- load k, q (bf16) and g (fp32) rows; rows past the end are zero
  {
    // rows past the end are read at the last valid row, then zeroed (branch-free loads)
    const int r = t >> 2, cb = t & 3;
    const bool ok = r < Cn;
    const int64_t e = ((tok0 + min(r, Cn - 1)) * H + h) * DK + cb * 32;
    u16x8 kv[4], qv[4], gv[4];
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) {
      kv[vv] = *reinterpret_cast<const u16x8*>(k + e + 8 * vv);
      qv[vv] = *reinterpret_cast<const u16x8*>(q + e + 8 * vv);
      gv[vv] = *reinterpret_cast<const u16x8*>(g + e + 8 * vv);
    }
    const uint16_t braw = beta[(tok0 + min(t & (C - 1), Cn - 1)) * H + h];
#pragma unroll
    for (int vv = 0; vv < 4; ++vv)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = cb * 32 + 8 * vv + i;
        Ks[r * KS + c] = ok ? kv[vv][i] : (uint16_t)0;
        Qs[r * KS + c] = ok ? qv[vv][i] : (uint16_t)0;
        Gs[r * GS + c] = ok ? bf16_bits_to_f32(gv[vv][i]) : 0.f;
      }
    if (t < C) Bs[t] = (t < Cn) ? bf16_bits_to_f32(braw) : 0.f;
  }
  __syncthreads();
  // ---- cumulative log-decay down the chunk, stored in log2 units
  if (t < DK) {
    float col[C];
#pragma unroll
    for (int r = 0; r < C; ++r) col[r] = Gs[r * GS + t];
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      acc += col[r];
      Gs[r * GS + t] = acc * kLog2e;
    }
  }
  __syncthreads();
  const int l = t & 63, gq = l >> 4, m = l & 15;
  // ---- e^{G_C}
  if (t < DK) reinterpret_cast<float*>(blk + OFF_GAM)[t] = exp2f(Gs[(C - 1) * GS + t]);
  // ---- Kbar, Qbar fragments: [ks][row tile]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int f = (t >> 6) + 4 * j;  // 0..15
    const int ks = f >> 2, mt = f & 3;
    const int row = 16 * mt + m;
    half8 kb, qb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = 32 * ks + kslot(gq, i);
      const float e = exp2f(Gs[row * GS + c]);
      kb[i] = static_cast<_Float16>(-bfv(Ks + row * KS + c) * e);
      qb[i] = static_cast<_Float16>(bfv(Qs + row * KS + c) * e);
    }
    *reinterpret_cast<half8*>(blk + OFF_KB + f * 1024 + l * 16) = kb;
    *reinterpret_cast<half8*>(blk + OFF_QB + f * 1024 + l * 16) = qb;
  }
  // ---- Ktil^T fragments: [dk tile][ks over chunk rows]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int f = (t >> 6) + 4 * j;
    const int mt = f >> 1, ks = f & 1;
    const int ch = 16 * mt + m;
    const float gC = Gs[(C - 1) * GS + ch];
    half8 kt;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 32 * ks + kslot(gq, i);
      kt[i] = static_cast<_Float16>(bfv(Ks + row * KS + ch) * exp2f(gC - Gs[row * GS + ch]));
    }
    *reinterpret_cast<half8*>(blk + OFF_KT + f * 1024 + l * 16) = kt;
  }
  // ---- A and Aqk on the matrix cores, wave w = row tile w
  floatx4 akk[4], aqk[4];
  const int w = t >> 6;
  switch (w) {
    case 0: tile_products<0>(Ks, Qs, Gs, l, akk, aqk); break;
    case 1: tile_products<1>(Ks, Qs, Gs, l, akk, aqk); break;
    case 2: tile_products<2>(Ks, Qs, Gs, l, akk, aqk); break;
    default: tile_products<3>(Ks, Qs, Gs, l, akk, aqk); break;
  }
  __syncthreads();  // Ks, Qs, Gs are dead from here on
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * gq + i, jc = 16 * b + m;
      A32[r * 64 + jc] = (b <= w && jc < r) ? Bs[r] * akk[b][i] : 0.f;
      AQ32[r * 64 + jc] = (b <= w && jc <= r) ? aqk[b][i] : 0.f;
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
      float s = 0.f;
#pragma unroll
      for (int mm = 0; mm < i; ++mm)
        if (mm >= j) s += A32[(o + i) * 64 + o + mm] * col[mm];
      col[i] = (i < j) ? 0.f : (i == j ? 1.f : -s);
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
  for (int j = 0; j < 2; ++j) {
    const int f = (t >> 6) + 4 * j;  // 0..7
    const int mt = f >> 1, ks = f & 1;
    const int row = 16 * mt + m;
    half8 mf, ah, al;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int cc = 32 * ks + kslot(gq, i);
      mf[i] = static_cast<_Float16>(T32[row * 64 + cc] * Bs[cc]);
      _Float16 hh, ll;
      split_f16(AQ32[row * 64 + cc], hh, ll);
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

template <typename TOut>
__global__ __launch_bounds__(256) void rec_kernel(
    const uint16_t* __restrict__ v, const float* __restrict__ S0, TOut* __restrict__ o,
    float* __restrict__ S_T, const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off,
    int T, int H, int n_seq, int64_t max_chunks, const uint8_t* __restrict__ ws) {
  // Two fp16 exchanges per chunk, double-buffered: the state strip (all 128 key rows) so
  // every wave can form complete Kbar S and Qbar S for its own 16 chunk rows, and
  // Y = V - Kbar S (all 64 chunk rows) for U' = M Y. Both are stored column-major
  // ([column][row]) so that the rows a lane needs for a B operand are contiguous, with
  // rows padded by 8 halves against bank conflicts.
  constexpr int SR = DK + 8, YR = C + 8;
  __shared__ __align__(16) _Float16 sx[2][16][SR];
  __shared__ __align__(16) _Float16 yx[2][16][YR];

  // XCD-aware placement: the 8 strips of one (sequence, head) share an XCD and its L2.
  const int b = blockIdx.x;
  const int xcd = b & 7, rest = b >> 3;
  const int strip = rest % NSTRIP;
  const int64_t pair = (int64_t)(rest / NSTRIP) * 8 + xcd;
  if (pair >= (int64_t)n_seq * H) return;
  const int n = (int)(pair / H), h = (int)(pair % H);
  const SeqInfo si = seq_info(n, cu, chunk_off, T);
  // a malformed cu_seqlens cannot make the chunk walk leave the workspace
  const int64_t nc = max((int64_t)0, min((si.len + C - 1) / C, max_chunks - si.cid0));

  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l = t & 63, gq = l >> 4, nn = l & 15;
  const int col = 16 * strip + nn;
  const int64_t s_base = pair * DK * DV;
  const int row_stride = H * DV;  // elements between consecutive tokens

  // this wave's state rows 32w + 16u + 4gq + i (u = 0, 1), column col
  floatx4 s[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s[u][i] = S0 ? S0[s_base + (int64_t)(32 * w + 16 * u + 4 * gq + i) * DV + col] : 0.f;

  // per-lane byte offsets, fixed for the whole sequence
  const int frag_off = l * 16;
  int v_off[4], o_off[4];  // this wave's chunk rows 16w + 4gq + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v_off[i] = ((16 * w + 4 * gq + i) * row_stride + col) * 2;
    o_off[i] = ((16 * w + 4 * gq + i) * row_stride + col) * (int)sizeof(TOut);
  }
  const int gam_off = OFF_GAM + (32 * w + 4 * gq) * 4;

  const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
  half8 kn[4], qb[4], mf[4][2], ahi[2], alo[2], kt[2][2];
  floatx4 gam[2];
  uint16_t vraw[4];

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

  auto load_kq = [&](rsrc_t r) {  // this wave's row tile, all four dk k-steps
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kn[j] = ld_frag(r, frag_off, OFF_KB + (j * 4 + w) * 1024);
      qb[j] = ld_frag(r, frag_off, OFF_QB + (j * 4 + w) * 1024);
    }
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
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) kt[u][ks] = ld_frag(r, frag_off, OFF_KT + ((2 * w + u) * 2 + ks) * 1024);
      gam[u] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, gam_off, 64 * u, 0));
    }
  };
  auto load_v = [&](int64_t c) {
    const rsrc_t r = make_rsrc(v_base + c * tok_step, rows_bytes(c, 2));
#pragma unroll
    for (int i = 0; i < 4; ++i) vraw[i] = __builtin_amdgcn_raw_buffer_load_b16(r, v_off[i], 0, 0);
  };

  if (nc > 0) {
    const rsrc_t r0 = make_rsrc(blk_base, (int64_t)kBlockBytes);
    load_kq(r0);
    load_m(r0);
    load_a(r0);
    load_kt(r0);
    load_v(0);
  }
  int buf = 0;
  for (int64_t c = 0; c < nc; ++c) {
    // operands of the next chunk are loaded right after their use in this one (the last
    // chunk reloads itself), unconditionally, so every load has a chunk's time to land
    const int64_t cn = min(c + 1, nc - 1);
    const rsrc_t rn = make_rsrc(blk_base + cn * blk_step, (int64_t)kBlockBytes);
    // -- all-gather the state strip in fp16
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      typedef _Float16 half4 __attribute__((ext_vector_type(4)));
      half4 hv;
#pragma unroll
      for (int i = 0; i < 4; ++i) hv[i] = static_cast<_Float16>(s[u][i]);
      *reinterpret_cast<half4*>(&sx[buf][nn][32 * w + 16 * u + 4 * gq]) = hv;
    }
    __syncthreads();
    // -- complete -Kbar S and Qbar S for this wave's 16 chunk rows
    floatx4 X = zero, QS = zero;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8 bs;
      const _Float16* sp = &sx[buf][nn][32 * j + 4 * gq];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bs[i] = sp[i];
        bs[i + 4] = sp[16 + i];
      }
      X = mfma_f16(kn[j], bs, X);
      QS = mfma_f16(qb[j], bs, QS);
    }
    load_kq(rn);
    // -- Y = V - Kbar S for this wave's rows, all-gathered in fp16
    {
      typedef _Float16 half4 __attribute__((ext_vector_type(4)));
      half4 hy;
#pragma unroll
      for (int i = 0; i < 4; ++i) hy[i] = static_cast<_Float16>(X[i] + bf16_bits_to_f32(vraw[i]));
      *reinterpret_cast<half4*>(&yx[buf][nn][16 * w + 4 * gq]) = hy;
    }
    load_v(cn);
    __syncthreads();
    // -- U' = M Y, all 64 rows (each wave keeps a full copy)
    floatx4 U[4];
    {
      half8 by[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const _Float16* yp = &yx[buf][nn][32 * ks + 4 * gq];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          by[ks][i] = yp[i];
          by[ks][i + 4] = yp[16 + i];
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        U[mt] = mfma_f16(mf[mt][0], by[0], zero);
        U[mt] = mfma_f16(mf[mt][1], by[1], U[mt]);
      }
    }
    load_m(rn);
    half8 uh[2], ul[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        _Float16 hh, ll;
        split_f16(i < 4 ? U[2 * ks][i] : U[2 * ks + 1][i - 4], hh, ll);
        uh[ks][i] = hh;
        ul[ks][i] = ll;
      }
    // -- outputs of this wave's rows: Qbar S + Aqk U'
    floatx4 acc = QS;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (ks == 1 && w < 2) break;  // Aqk is lower triangular: rows < 32 see k-step 0 only
      acc = mfma_f16(ahi[ks], uh[ks], acc);
      acc = mfma_f16(ahi[ks], ul[ks], acc);
      acc = mfma_f16(alo[ks], uh[ks], acc);
    }
    load_a(rn);
    {
      const rsrc_t ro = make_rsrc(o_base + c * tok_step, rows_bytes(c, (int)sizeof(TOut)));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (sizeof(TOut) == 4)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i]), ro, o_off[i], 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(acc[i]), ro, o_off[i], 0, 0);
      }
    }
    // -- this wave's state rows: S = Diag(e^{G_C}) S + Ktil^T U'
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      s[u] *= gam[u];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        s[u] = mfma_f16(kt[u][ks], uh[ks], s[u]);
        s[u] = mfma_f16(kt[u][ks], ul[ks], s[u]);
      }
    }
    load_kt(rn);
    buf ^= 1;
  }
  if (S_T) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S_T[s_base + (int64_t)(32 * w + 16 * u + 4 * gq + i) * DV + col] = s[u][i];
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
  const int64_t rec_blocks = ((pairs + 7) / 8) * 8 * NSTRIP;
  if (p.out_bf16)
    hipLaunchKernelGGL(rec_kernel<uint16_t>, dim3((unsigned)rec_blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(p.v), p.S0, static_cast<uint16_t*>(p.o),
                       p.S_T, p.cu_seqlens, chunk_off, p.T, p.H, p.n_seq, max_chunks(p), ws);
  else
    hipLaunchKernelGGL(rec_kernel<float>, dim3((unsigned)rec_blocks), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(p.v), p.S0, static_cast<float*>(p.o), p.S_T,
                       p.cu_seqlens, chunk_off, p.T, p.H, p.n_seq, max_chunks(p), ws);
  return hipGetLastError();
}

}  // namespace kda
