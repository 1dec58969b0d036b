// Matrix-core chunked KDA forward for gfx950: bf16 activations, dk = dv = 128, chunk 64.
//
// The chunked algebra (from the recurrence S_r = (I - b_r k_r k_r^T) D_r S_{r-1} + b_r k_r v_r^T)
// for a 64-token chunk entered with state S, G_r = sum_{j<=r} g_j per key channel:
//   U' = M (V - Kbar S) = Utilde - W S,   M = (I + A)^{-1} diag(b),  W = M Kbar,  Utilde = M V
//   A[r][j] = b_r sum_c k_r k_j e^{G_r - G_j} (j < r),   Aqk[r][j] = sum_c q_r k_j e^{G_r - G_j} (j <= r)
//   O  = Qbar S + Aqk U' = Qhat S + Ohat,   Qhat = Qbar - P Kbar,   Ohat = P V,   P = Aqk M
//   S <- Diag(e^{G_C}) S + Ktil^T U' = Diag(e^{G_C}) S + Z - Phi S = S + Z + Psi S,
//   Phi = Ktil^T W,  Z = Ktil^T Utilde,  Psi = -Phi - Diag(1 - e^{G_C})
// with Kbar = K e^{G}, Qbar = Q e^{G}, Ktil = K e^{G_C - G}. Everything that does not depend on
// the entry state (Psi, Z, Qhat, Ohat) is formed for all chunks in parallel; the serial walk
// over the chunks then needs two products with the state per chunk (Psi S for the update,
// Qhat S for the outputs), both of the state as it enters the chunk, so one exchange of the
// state between waves per chunk suffices. Folding the decay into Psi (fp16) costs no
// precision where it matters: the stored diagonal term is 1 - e^{G_C}, small exactly when the
// state is carried over many chunks, while the carried state itself stays in fp32.
//
// Two kernels.
//  prep_kernel (one workgroup per chunk and head, all chunks in parallel): the per-channel
//    cumulative log-decay; A and Aqk on the matrix cores; the inverse (I + A)^{-1} by
//    blocked forward substitution in LDS; then P, Qhat, Ohat, W, Utilde, Psi and Z on the
//    matrix cores. Channel-major (transposed) operands come from products with an identity
//    fragment, so no LDS staging array is needed.
//    Results are stored in the workspace already in MFMA lane order, so each later load is
//    one coalesced 16-byte load per lane: operand "fragments" (1 KiB = 64 lanes x 8 fp16)
//    and result tiles (1 KiB = 64 lanes x 4 fp32).
//    A and Aqk are built from 16-token tiles whose exponent is measured from the state before
//    the row tile: the row factor e^{G_r - ref} lies in [e^-80, 1] and the column factor
//    e^{ref - G_j} is <= 1 off the diagonal and in [1, e^80] on it, because each step's
//    log-decay is >= -5 (orkas.ai Kimi K3 page, "Eine Untergrenze, die einen GPU-Codepfad
//    beseitigte"). The diagonal tiles therefore run the same dense MFMA as the others; their
//    operands need bf16's exponent range (fp16 would overflow at e^80), and are split into
//    bf16 hi + lo pairs (three products) to keep 16 bits of precision. Off-diagonal factors
//    are <= 1 and use fp16 (11-bit significand) directly.
//  rec_kernel (one workgroup per sequence, head and strip of 16, 32 or 64 value columns,
//    serial over chunks): the fp32 state slice S[128][16 .. 64] lives in MFMA accumulators for
//    the whole sequence. Eight waves in two roles. Waves 0-3 own 32 key rows of the state each
//    and carry the dependency chain: S <- S + Z + Psi S for their rows. Waves 4-7 compute the
//    outputs Qhat S + Ohat of their 16 chunk rows from the same gathered state, off the chain.
//    Columns of S evolve independently (the transition acts on the key side only), so
//    splitting the value columns over workgroups is exact. When the walks would leave half of
//    the CUs idle, two workgroups repeat each walk and split its output rows; packed
//    sequences are walked longest first.
// With few (sequence, head) pairs the walk's serial latency dominates, and one step of the
// walk covers two chunks a, b: a prep workgroup of eight waves forms both chunks (four waves
// each) and composes them, S -> S + Z' + Psi' S with Psi' = Psi_a + Psi_b + Psi_b Psi_a and
// Z' = Z_a + Z_b + Psi_b Z_a, chunk b's outputs reading the state entering the pair through
// Qhat_b (I + Psi_a) and Ohat_b + Qhat_b Z_a. Half the steps, and Psi' and Z' stored once
// per 128 tokens.
// With many pairs the walk streams its operands at what HBM delivers, and the block is stored
// factored instead (W, Ktil^T, Utilde, Qbar, Aqk, e^{G_C}: 14 % fewer bytes, and prep skips
// P, Qhat, Ohat, Phi and Z): rec_fact_kernel then forms U' = Utilde - W S per chunk and takes
// both the state update and the outputs from it, with two exchanges per chunk instead of one.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_plan.h"

namespace kda {

namespace {

constexpr int C = 64;
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int NSTRIP = DV / 16;  // 16-column strips per (sequence, head)

// Workspace block of BL tokens of one head, byte offsets: BL = 64 holds one chunk, BL = 128
// two consecutive chunks composed into one step of the walk. Fragment f of a group starts at
// group + f * 1024 (lane l's eight fp16 at + l * 16); a result tile f likewise (four fp32).
//   phi  Psi as A operand: [key row tile (8)][k-step over keys (4)]                 32 KiB
//   qh   Qhat as A operand: [k-step over dk (4)][row tile (BL / 16)]      4 KiB per row tile
//   z    Z, fp16 tiles in accumulator layout:
//        [value tile (8)][key row pair (4)][lane][tile of the pair][4]              32 KiB
//   oh   Ohat result tiles, fp32: [value tile (8)][row tile (BL / 16)]    8 KiB per row tile
// Ohat stays fp32: the largest outputs reach tens of times their RMS, and fp16 rounding of
// Ohat alone put half of the 2e-2 max-abs budget on the long workloads.
struct Layout {
  int phi, qh, z, oh, block;
};
constexpr Layout layout(int BL) {
  return Layout{0, 32768, 32768 + (BL / 16) * 4096, 65536 + (BL / 16) * 4096,
                65536 + (BL / 16) * 12288};
}
static_assert(layout(64).block == 114688 && layout(128).block == 163840, "block sizes");

// Factored block of one 64-token chunk (byte offsets): the walk forms U' = Utilde - W S itself
// and takes both the state update and the outputs from it.
//   w    W as A-operand fragments [token row tile rt][key k-step j]            16 KiB
//   kt   Ktil^T as A-operand fragments [key row tile kt][token k-step jt]      16 KiB
//   ut   Utilde fp32 result tiles [value tile ct][token row tile rt]           32 KiB
//   qb   Qbar as A-operand fragments [key k-step j][token row tile rt]         16 KiB
//   ah   Aqk high fp16 part, A-operand fragments [token k-step jt][row tile rt]  8 KiB
//   al   Aqk low fp16 part, same order                                           8 KiB
//   gam  e^{G_C} per key channel, fp32                                          512 B
struct FLayout {
  int w, kt, ut, qb, ah, al, gam, block;
};
constexpr FLayout flayout() { return FLayout{0, 16384, 32768, 65536, 81920, 90112, 98304, 98816}; }

struct SeqInfo {
  int64_t tok0;  // first token of the sequence in the packed T axis
  int64_t len;
  int64_t cid0;  // first block of the sequence in the workspace
};

// sequence n's tokens, and its first workspace block of BL tokens
template <int BL>
__device__ __forceinline__ SeqInfo seq_info(int n, const int32_t* cu, const int32_t* blk_off,
                                            int T) {
  SeqInfo s;
  if (cu) {
    const int64_t a = min(max((int64_t)cu[n], (int64_t)0), (int64_t)T);
    const int64_t e = min(max((int64_t)cu[n + 1], a), (int64_t)T);
    s.tok0 = a;
    s.len = e - a;
    s.cid0 = blk_off[n];
  } else {
    s.tok0 = (int64_t)n * T;
    s.len = T;
    s.cid0 = (int64_t)n * ((T + BL - 1) / BL);
  }
  return s;
}

// blk_off[n] = number of blocks of blk_len tokens of sequences 0..n-1 (lengths clamped as in
// seq_info), and,
// when every > 0, ckpt_off[n] = number of state checkpoints of sequences 0..n-1 (one per full
// `every` tokens of each). order[] lists the sequences longest first (ties by index) when
// there are at most kMaxOrdered of them, else in their own order: the walks are then
// dispatched longest first, so the longest ones do not start last and set the tail.
constexpr int kMaxOrdered = 512;
__global__ __launch_bounds__(256) void plan_kernel(const int32_t* __restrict__ cu, int n_seq,
                                                   int T, int blk_len, int every,
                                                   int32_t* __restrict__ blk_off,
                                                   int32_t* __restrict__ ckpt_off,
                                                   int32_t* __restrict__ order) {
  __shared__ int64_t part[2][256];
  const int t = threadIdx.x;
  const int per = (n_seq + 255) / 256;
  const int lo = min(t * per, n_seq), hi = min(lo + per, n_seq);
  auto seq_len = [&](int n) {
    const int64_t a = min(max((int64_t)cu[n], (int64_t)0), (int64_t)T);
    const int64_t e = min(max((int64_t)cu[n + 1], a), (int64_t)T);
    return e - a;
  };
  int64_t sum = 0, sck = 0;
  for (int n = lo; n < hi; ++n) {
    const int64_t len = seq_len(n);
    sum += (len + blk_len - 1) / blk_len;
    if (every > 0) sck += len / every;
  }
  part[0][t] = sum;
  part[1][t] = sck;
  __syncthreads();
  if (t < 2) {
    int64_t acc = 0;
    for (int i = 0; i < 256; ++i) {
      const int64_t x = part[t][i];
      part[t][i] = acc;
      acc += x;
    }
  }
  __syncthreads();
  int64_t acc = part[0][t], ack = part[1][t];
  for (int n = lo; n < hi; ++n) {
    const int64_t len = seq_len(n);
    blk_off[n] = (int32_t)acc;
    acc += (len + blk_len - 1) / blk_len;
    if (every > 0) {
      ckpt_off[n] = (int32_t)ack;
      ack += len / every;
    }
  }
  if (t == 255) blk_off[n_seq] = (int32_t)acc;
  for (int n = lo; n < hi; ++n) {  // the rank of n is its slot: a permutation of 0..n_seq-1
    int rank = n;
    if (n_seq <= kMaxOrdered) {
      const int64_t len = seq_len(n);
      rank = 0;
      for (int m = 0; m < n_seq; ++m) {
        const int64_t lm = seq_len(m);
        rank += (lm > len || (lm == len && m < n)) ? 1 : 0;
      }
    }
    order[rank] = n;
  }
}

// ---------------------------------------------------------------- prep
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes): loads past the end return zero and stores
// past the end are dropped, which is how partial chunks are masked without branches.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = (int)min(max(bytes, (int64_t)0), (int64_t)0x7fffffff);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
// Workspace stores of 16 bytes per lane are global stores: a buffer store wider than 8 bytes
// with an SGPR offset gets no wait state before its data registers are rewritten, and on
// gfx950 the last dword of some lanes was then read after the rewrite (wrong workspace values,
// intermittently).

// 2^x for x in [-116, 0], the range of a decay factor across one 16-token tile (each step's
// log-decay is >= -5): the hardware exp2 is exact to its ulp bound there and needs none of
// the scaling that exp2f adds for arguments below -126.
__device__ __forceinline__ float exp2_tile(float x) { return __builtin_amdgcn_exp2f(x); }
// Eight fp32 values split into bf16 hi (nearest) + lo (the nearest bf16 to the residual), two
// values per conversion; hi is widened back by shifting its halves into place.
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  u32x4 h, r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t hu = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[2 * i], x[2 * i + 1]}, bf16x2));
    const float h0 = __uint_as_float(hu << 16), h1 = __uint_as_float(hu & 0xffff0000u);
    h[i] = hu;
    r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[2 * i] - h0, x[2 * i + 1] - h1}, bf16x2));
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ half8 frag_from_halves(const half4& a, const half4& b) {
  half8 f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = a[i];
    f[i + 4] = b[i];
  }
  return f;
}
// Fragment (rows r, K slots of a 32-wide k-step) from a [row][k] fp16 array: slot i < 4 is
// k = 4 gq + i, slot i >= 4 is k = 16 + 4 gq + i - 4.
__device__ __forceinline__ half8 lds_frag(const _Float16* rowp, int gq) {
  return frag_from_halves(*reinterpret_cast<const half4*>(rowp + 4 * gq),
                          *reinterpret_cast<const half4*>(rowp + 16 + 4 * gq));
}

// One workgroup per (chunk, head); wave a owns row tile a (chunk rows 16a .. 16a+15). In the
// MFMA fragment layout lane l of wave a holds row 16a + (l & 15) and, for each of the four
// 32-channel k-steps, the eight channels 32 ks + kslot(l >> 4, i). The per-tile cumulative
// decay is a prefix sum over the tile's 16 rows, formed on the matrix cores in that same
// layout. Every per-element quantity is formed once, in registers, in that layout:
//   rf = e^{G_r - ref_a}   (ref_a = G at the last token before tile a)   in [e^-80, 1]
//   cf = e^{Gend_a - G_r}  (Gend_a = G at the last token of tile a)       in [e^-80, 1]
// The row operand of tile a is k rf (q rf), its diagonal column operand k / rf (in [1, e^80]
// times k, bf16 range), and the column operand it lends to later tiles b > a is k cf, scaled
// there by the per-channel factor e^{ref_b - Gend_a} <= 1. Kbar, Qbar and Ktil follow from the
// same values times per-channel constants. Products are arranged so that their results land
// in the lane layout the next product or the workspace needs: a result tile computed as
// (column operand) x (row operand) leaves each lane with four entries of its own row, which
// for two adjacent tiles is exactly an A-operand fragment of that row.
// PAIRWISE replaces the dense diagonal tiles by the pairwise evaluation of the earlier
// generation (each e^{G_r - G_j} formed per pair and channel, in fp32 on the vector ALUs),
// which needs no bound on the decay: the ablation that measures what the bound buys.
template <bool PAIRWISE, bool COMPOSE, bool FACT = false>
__global__ __launch_bounds__(COMPOSE ? 512 : 256, 2) void prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ beta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ blk_off, int T, int H,
    int n_seq, uint8_t* __restrict__ ws) {
  constexpr int BL = COMPOSE ? 2 * C : C;  // tokens per workspace block
  constexpr int NGRP = COMPOSE ? 2 : 1;    // groups of four waves, one chunk each
  constexpr Layout LY = layout(BL);
  constexpr int AS = C + 4;  // row stride (fp32) of A and T
  // One LDS arena reused phase by phase (byte ranges), 66 KB, two workgroups per CU (the
  // kernel needs about 190 registers; at three workgroups it spilled, and every spill reload
  // waited for all loads in flight):
  //   tile products: lent column operands k cf, fp32 [3][4][64][8]     [0, 24576)
  //                  per-channel tables (tile totals and factors)     [24576, 32256)
  //                  Kbar^T fragments (kept until the last products)  [34816, 51200)
  //                  Ktil^T fragments (kept until the last products)  [51200, 67584)
  //   inverse:       A fp32 [64][AS] [0, 17408), T [17408, 34816)
  //   products:      V fragments [0, 16384), once M and P are in registers
  // A fragment array holds 16 fragments [16-column tile][k-step over chunk rows], each in
  // MFMA operand order (64 lanes x 8 fp16).
  // The pairwise ablation first stages per wave G fp32 [16][132] and k, q bf16 [16][136].
  constexpr int PW_G = 16 * 132 * 4, PW_KQ = 16 * 136 * 2, PW_WAVE = PW_G + 2 * PW_KQ;
  constexpr int OFF_TAB = PAIRWISE ? 4 * PW_WAVE : 24576;
  constexpr int OFF_KBF = 34816, OFF_KTL = 51200;
  constexpr int ARENA = PAIRWISE ? OFF_TAB + 7680 : 67584;
  __shared__ __align__(16) unsigned char arenas[NGRP][ARENA];
  __shared__ __align__(16) float Bss[NGRP][C];
  __shared__ float GAMSS[NGRP][DK];  // e^{G_C} per key channel, for the diagonal of Psi

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int grp = wave >> 2;  // which chunk of the block this wave works on
  const int w = wave & 3;
  unsigned char* arena = arenas[grp];
  float* Bs = Bss[grp];
  float* GAMS = GAMSS[grp];
  float* KC = reinterpret_cast<float*>(arena);
  float(*TOT)[DK] = reinterpret_cast<float(*)[DK]>(arena + OFF_TAB);
  float(*PCH)[DK] = reinterpret_cast<float(*)[DK]>(arena + OFF_TAB + 2048);
  float(*ECH)[DK] = reinterpret_cast<float(*)[DK]>(arena + OFF_TAB + 4096);
  float(*XCH)[DK] = reinterpret_cast<float(*)[DK]>(arena + OFF_TAB + 6144);
  half8* KBF = reinterpret_cast<half8*>(arena + OFF_KBF);
  half8* KTL = reinterpret_cast<half8*>(arena + OFF_KTL);
  float* A32 = reinterpret_cast<float*>(arena);
  float* T32 = reinterpret_cast<float*>(arena + 17408);
  half8* VBF = reinterpret_cast<half8*>(arena);
  static_assert(!PAIRWISE || OFF_TAB + 7680 <= ARENA, "layout");
  static_assert(OFF_KTL + 16384 <= ARENA && (PAIRWISE || OFF_TAB + 7680 <= OFF_KBF), "layout");
  static_assert(4 * PW_WAVE <= (PAIRWISE ? ARENA : 1 << 30), "layout");

  // one workgroup per (block, head); the whole workgroup leaves together, so that the
  // barriers below always see every wave
  const int h = blockIdx.x % H;
  const int64_t bid = blockIdx.x / H;
  int n;
  int64_t b_in;
  if (cu) {
    if (bid >= blk_off[n_seq]) return;
    int lo = 0, hi = n_seq - 1;  // last n with blk_off[n] <= bid
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (blk_off[mid] <= bid) lo = mid; else hi = mid - 1;
    }
    n = lo;
    b_in = bid - blk_off[n];
  } else {  // dense batch
    const int64_t nbs = (T + BL - 1) / BL;
    n = (int)(bid / nbs);
    b_in = bid % nbs;
    if (n >= n_seq) return;
  }
  const SeqInfo si = seq_info<BL>(n, cu, blk_off, T);
  // this group's chunk; the second chunk of a sequence's last block may hold no token (then
  // every load below reads zero and the chunk is the identity transition)
  const int64_t c_in = b_in * NGRP + grp;
  const int64_t tok0 = si.tok0 + c_in * C;
  const int Cn = (int)max((int64_t)0, min((int64_t)C, si.len - c_in * C));
  static_assert(!(FACT && COMPOSE), "the factored block is one chunk");
  uint8_t* blk = ws + ((size_t)(si.cid0 + b_in) * H + h) * (FACT ? flayout().block : LY.block);

  const int l = t & 63, gq = l >> 4, m = l & 15;
  const int row = 16 * w + m;

  // ---- this lane's 32 elements of row 16w + m of k, q, g, v. The loads go through buffer
  //      resources that end after the chunk's last valid row, so rows past the end read as
  //      zero (k = q = v = 0, g = 0: decay 1, beta = 0) with no mask on the values.
  u16x4 kraw[4][2], qraw[4][2], graw[4][2], vraw[4][2];
  uint16_t braw;
  const int64_t tok_elems = (int64_t)H * DK;  // elements between consecutive tokens
  const int64_t e0 = (tok0 * H + h) * DK;
  const int64_t valid = ((int64_t)(Cn - 1) * tok_elems + DK) * 2;
  const rsrc_t rs_q = make_rsrc(q + e0, valid), rs_k = make_rsrc(k + e0, valid),
               rs_g = make_rsrc(g + e0, valid), rs_v = make_rsrc(v + e0, valid);
  const int in_off = (int)((row * tok_elems + 4 * gq) * 2);
  auto ld_in = [&](rsrc_t r, int ks, int hf) {
    return __builtin_bit_cast(u16x4, __builtin_amdgcn_raw_buffer_load_b64(r, in_off, (32 * ks + 16 * hf) * 2, 0));
  };
  {
    // g first: the decay scan needs only g, and loads complete in the order they are issued,
    // so the scan waits for a third of the bytes while k and q are still arriving. q of the
    // last two k-steps is loaded during the tile products, two k-steps ahead of its use
    // (fewer registers held through the column pass; measured faster than loading it here).
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        graw[ks][hf] = ld_in(rs_g, ks, hf);
    braw = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(beta + tok0 * H + h, ((int64_t)(Cn - 1) * H + 1) * 2),
                                                row * H * 2, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // keep the issue order
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        kraw[ks][hf] = ld_in(rs_k, ks, hf);
#pragma unroll
    for (int ks = 0; ks < (PAIRWISE ? 4 : 2); ++ks)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        qraw[ks][hf] = ld_in(rs_q, ks, hf);
    __builtin_amdgcn_sched_barrier(0);
  }
  // ---- cumulative log-decay within the row tile (log2 units), on the matrix cores. The
  //      identity product turns each 16-channel half of a k-step of g channel-major (a lane then
  //      holds four rows of one channel; exact: bf16 values times one); the product of that with
  //      the transposed 16 x 16 lower triangle of ones, g^T L^T, is every row's inclusive prefix
  //      sum, in the inputs' own layout (row m, channels 16 hf + 4 gq + i).
  float gsa[4][8];
  {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x8 idb[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        idb[hf][i] = static_cast<__bf16>((i >> 2) == hf && 4 * gq + (i & 3) == m ? 1.f : 0.f);
    bf16x4 ltri;  // L^T: rows 4 gq + i, column m
#pragma unroll
    for (int i = 0; i < 4; ++i) ltri[i] = static_cast<__bf16>(4 * gq + i <= m ? 1.f : 0.f);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 gf = __builtin_bit_cast(bf16x8, u16x8{graw[ks][0][0], graw[ks][0][1], graw[ks][0][2], graw[ks][0][3],
                                                         graw[ks][1][0], graw[ks][1][1], graw[ks][1][2], graw[ks][1][3]});
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const floatx4 tr = mfma_bf16(gf, idb[hf], floatx4{0.f, 0.f, 0.f, 0.f});
        bf16x4 gt;
#pragma unroll
        for (int i = 0; i < 4; ++i) gt[i] = static_cast<__bf16>(tr[i]);
        const floatx4 d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(gt, ltri, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) gsa[ks][4 * hf + i] = d[i] * kLog2e;
      }
    }
  }
  auto scan_ks = [&](int ks, float (&gk)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) gk[i] = gsa[ks][i];
  };
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    float gk[8];
    scan_ks(ks, gk);
    if (m == 15) {  // the tile's totals
      *reinterpret_cast<floatx4*>(&TOT[w][32 * ks + 4 * gq]) = floatx4{gk[0], gk[1], gk[2], gk[3]};
      *reinterpret_cast<floatx4*>(&TOT[w][32 * ks + 16 + 4 * gq]) = floatx4{gk[4], gk[5], gk[6], gk[7]};
    }
  }
  if (gq == 0) Bs[row] = bf16_bits_to_f32(braw);
  __syncthreads();
  // ---- per-channel constants from the tile totals (half the threads per pair of tiles)
  {
    const int c = t & (DK - 1), hf = (t >> 7) & 1;  // this group's 256 threads
    const float t0 = TOT[0][c], t1 = TOT[1][c], t2 = TOT[2][c], t3 = TOT[3][c];
    const float ref[4] = {0.f, t0, t0 + t1, t0 + t1 + t2};
    const float tt[4] = {t0, t1, t2, t3};
    const float gc = ref[3] + t3;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if ((a >> 1) != hf) continue;
      PCH[a][c] = exp2f(ref[a]);               // e^{ref_a}: Kbar = (k rf) e^{ref_a}
      ECH[a][c] = exp2f(gc - (ref[a] + tt[a]));  // e^{G_C - Gend_a}: Ktil = (k cf) e^{G_C - Gend_a}
    }
    if (hf == 0) {
      XCH[0][c] = exp2f(t1);       // column factor of block (2, 0): e^{ref_2 - Gend_0}
      XCH[1][c] = exp2f(t1 + t2);  // (3, 0)
      GAMS[c] = exp2f(gc);
    } else {
      XCH[2][c] = exp2f(t2);       // (3, 1)
    }
  }
  __syncthreads();
  // ---- pairwise diagonal tile (ablation): lane (row n = m, columns 4 gq + i) forms
  //      A[r][j] = sum_c k_r k_j e^{G_r - G_j} and Aqk[r][j] over its four columns j <= r
  floatx4 pw_k = {0.f, 0.f, 0.f, 0.f}, pw_q = pw_k;
  if constexpr (PAIRWISE) {
    float* Gw = reinterpret_cast<float*>(arena + w * PW_WAVE);
    uint16_t* Kw = reinterpret_cast<uint16_t*>(arena + w * PW_WAVE + PW_G);
    uint16_t* Qw = reinterpret_cast<uint16_t*>(arena + w * PW_WAVE + PW_G + PW_KQ);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float gk[8];
      scan_ks(ks, gk);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int c0 = 32 * ks + 16 * hf + 4 * gq;
        *reinterpret_cast<floatx4*>(&Gw[m * 132 + c0]) =
            floatx4{gk[4 * hf], gk[4 * hf + 1], gk[4 * hf + 2], gk[4 * hf + 3]};
        *reinterpret_cast<u16x4*>(&Kw[m * 136 + c0]) = kraw[ks][hf];
        *reinterpret_cast<u16x4*>(&Qw[m * 136 + c0]) = qraw[ks][hf];
      }
    }
    __syncthreads();
    for (int c = 0; c < DK; c += 4) {
      const floatx4 gr = *reinterpret_cast<const floatx4*>(&Gw[m * 132 + c]);
      const u16x4 kr4 = *reinterpret_cast<const u16x4*>(&Kw[m * 136 + c]);
      const u16x4 qr4 = *reinterpret_cast<const u16x4*>(&Qw[m * 136 + c]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * gq + i;
        const floatx4 gj = *reinterpret_cast<const floatx4*>(&Gw[j * 132 + c]);
        const u16x4 kj4 = *reinterpret_cast<const u16x4*>(&Kw[j * 136 + c]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // G_r - G_j <= 0 for j <= r; for j > r the term is discarded below
          const float f = bf16_bits_to_f32(kj4[e]) * exp2f(fminf(gr[e] - gj[e], 0.f));
          pw_k[i] = fmaf(bf16_bits_to_f32(kr4[e]), f, pw_k[i]);
          pw_q[i] = fmaf(bf16_bits_to_f32(qr4[e]), f, pw_q[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * gq + i > m) pw_k[i] = pw_q[i] = 0.f;
    __syncthreads();  // the arena is reused below
  }
  // identity fragments: as the B operand, idf[hf] copies channel tile hf of a 32-channel
  // k-step, so (row fragment) x idf[hf] is the row tile's 16 x 16 block with each lane holding
  // four rows of one channel, i.e. half of a channel-major (transposed) fragment. Exact: every
  // product is a value times one or zero.
  half8 idf[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      idf[hf][i] = static_cast<_Float16>((i >> 2) == hf && 4 * gq + (i & 3) == m ? 1.f : 0.f);
  // half-fragment slot of this wave's 16 rows in a transposed fragment [tile ct][k-step w / 2]:
  // byte ct * 2048 + half_lane
  const int half_lane = ((w >> 1) * 64 + l) * 16 + (w & 1) * 8;
  auto to_half4 = [](const floatx4& d) {
    half4 hv;
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = static_cast<_Float16>(d[i]);
    return hv;
  };
  auto store_half_lds = [&](uint8_t* base, int ct, const floatx4& d) {
    *reinterpret_cast<half4*>(base + ct * 2048 + half_lane) = to_half4(d);
  };
  const floatx4 zero = {0.f, 0.f, 0.f, 0.f};

  // ---- column operands: k cf lent to later row tiles, and Ktil^T fragments (LDS)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    float gk[8];
    scan_ks(ks, gk);
    floatx4 kc[2];
    half8 kt16;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int c0 = 32 * ks + 16 * hf + 4 * gq;
      const floatx4 tw = *reinterpret_cast<const floatx4*>(&TOT[w][c0]);
      const floatx4 ee = *reinterpret_cast<const floatx4*>(&ECH[w][c0]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float kv = bf16_bits_to_f32(kraw[ks][hf][j]);
        kc[hf][j] = kv * exp2_tile(tw[j] - gk[4 * hf + j]);  // k e^{Gend_w - G_r}
        kt16[4 * hf + j] = static_cast<_Float16>(kc[hf][j] * ee[j]);
      }
    }
    if (w < 3) {
      float* kcp = KC + ((w * 4 + ks) * 64 + l) * 8;
      *reinterpret_cast<floatx4*>(kcp) = kc[0];
      *reinterpret_cast<floatx4*>(kcp + 4) = kc[1];
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      store_half_lds(reinterpret_cast<uint8_t*>(KTL), 2 * ks + hf, mfma_f16(kt16, idf[hf], zero));
  }
  __syncthreads();
  // ---- per k-step: row factors, Qbar, Kbar^T fragments (LDS), and the A and Aqk tiles of row
  //      tile w. Each tile is computed as (column operand) x (row operand), i.e. transposed,
  //      so lane l ends with entries (16w + l&15, 16bb + 4 gq + i).
  floatx4 akk[3], aqk[3];
  // the diagonal tile has accumulators of its own, so that no register array is indexed by the
  // (run-time) wave number
  floatx4 akd = pw_k, aqd = pw_q;
#pragma unroll
  for (int bb = 0; bb < 3; ++bb) akk[bb] = aqk[bb] = zero;
  half8 qbar[4];  // Qbar as A-operand fragments of row tile w
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (!PAIRWISE && ks < 2) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        qraw[ks + 2][hf] = ld_in(rs_q, ks + 2, hf);
    }
    float gk[8];
    scan_ks(ks, gk);
    float kr[8], qr[8], kd[8];
    half8 kb16;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const floatx4 pe = *reinterpret_cast<const floatx4*>(&PCH[w][32 * ks + 16 * hf + 4 * gq]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * hf + j;
        const float kv = bf16_bits_to_f32(kraw[ks][hf][j]);
        const float qv = bf16_bits_to_f32(qraw[ks][hf][j]);
        const float rf = exp2_tile(gk[i]);  // e^{G_r - ref_w}
        kr[i] = kv * rf;
        qr[i] = qv * rf;
        kd[i] = kv * __builtin_amdgcn_rcpf(rf);
        qbar[ks][i] = static_cast<_Float16>(qr[i] * pe[j]);
        kb16[i] = static_cast<_Float16>(kr[i] * pe[j]);
      }
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      store_half_lds(reinterpret_cast<uint8_t*>(KBF), 2 * ks + hf, mfma_f16(kb16, idf[hf], zero));
    half8 rk16, rq16;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      rk16[i] = static_cast<_Float16>(kr[i]);
      rq16[i] = static_cast<_Float16>(qr[i]);
    }
    bf16x8 rkh, rkl, rqh, rql, ch, cl;
    split_bf16x8(kr, rkh, rkl);
    split_bf16x8(qr, rqh, rql);
    split_bf16x8(kd, ch, cl);
    // diagonal tile: column factor up to e^80, split bf16
    if constexpr (!PAIRWISE) {
      akd = mfma_bf16(ch, rkh, akd);
      akd = mfma_bf16(ch, rkl, akd);
      akd = mfma_bf16(cl, rkh, akd);
      aqd = mfma_bf16(ch, rqh, aqd);
      aqd = mfma_bf16(ch, rql, aqd);
      aqd = mfma_bf16(cl, rqh, aqd);
    }
    // earlier tiles: factors <= 1, fp16
#pragma unroll
    for (int bb = 0; bb < 3; ++bb) {
      if (bb >= w) break;
      const float* kcp = KC + ((bb * 4 + ks) * 64 + l) * 8;
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
      akk[bb] = mfma_f16(c16, rk16, akk[bb]);
      aqk[bb] = mfma_f16(c16, rq16, aqk[bb]);
    }
  }
  // v is first needed after the inverse: its load latency overlaps the substitution
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      vraw[ks][hf] = ld_in(rs_v, ks, hf);
  __syncthreads();  // the lent operands and the tables are dead: A and T take the arena
  // ---- beta-scaled A rows into LDS (entries on or above the diagonal are never read);
  //      Aqk (lower, diagonal included) as A-operand fragments hi + lo in registers
  {
    const float br = Bs[row];
#pragma unroll
    for (int bb = 0; bb < 3; ++bb)
      if (bb < w) *reinterpret_cast<floatx4*>(&A32[row * AS + 16 * bb + 4 * gq]) = br * akk[bb];
    *reinterpret_cast<floatx4*>(&A32[row * AS + 16 * w + 4 * gq]) = br * akd;
  }
  half8 ahi[2], alo[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int bb = 2 * ks + (i >> 2), ii = i & 3;
      const float a = bb < w ? aqk[bb < 3 ? bb : 2][ii] : (bb == w && 4 * gq + ii <= m) ? aqd[ii] : 0.f;
      _Float16 hh, ll;
      split_f16(a, hh, ll);
      ahi[ks][i] = hh;
      alo[ks][i] = ll;
    }
  __syncthreads();
  // ---- T = (I + A)^{-1}: diagonal 16x16 blocks by substitution (wave w, lane = column)
  if (l < 16) {
    const int j = l, o = 16 * w;
    // entries of column j above the diagonal are zero, so every term of the substitution
    // can be summed unconditionally (row values are the same for all lanes)
    float col[16];
    col[0] = j == 0 ? 1.f : 0.f;
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      const float* arow = A32 + (o + i) * AS + o;
      float sacc = 0.f;
#pragma unroll
      for (int mm = 0; mm < i; ++mm) sacc = fmaf(arow[mm], col[mm], sacc);
      col[i] = i == j ? 1.f : -sacc;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) T32[(o + i) * AS + o + j] = col[i];
  }
  __syncthreads();
  // ---- off-diagonal blocks, by distance L from the diagonal, on the fp32 matrix cores:
  //      T_ab = -T_aa * sum_{c=b}^{a-1} A_ac T_cb; at distance L wave w < 4 - L takes block
  //      (w + L, w). v_mfma_f32_16x16x4_f32 contracts four indices per step; step s uses
  //      k = 4 (l >> 4) + s, so the accumulator X (lane: rows 4 (l >> 4) + i of column l & 15)
  //      is directly the B operand of the product with T_aa.
#pragma unroll
  for (int L = 1; L < 4; ++L) {
    if (w < 4 - L) {
      const int a = w + L, bb = w;
      floatx4 X = zero;
      for (int cc = bb; cc < a; ++cc) {
        const floatx4 av = *reinterpret_cast<const floatx4*>(&A32[(16 * a + m) * AS + 16 * cc + 4 * gq]);
#pragma unroll
        for (int st = 0; st < 4; ++st)
          X = __builtin_amdgcn_mfma_f32_16x16x4f32(av[st], T32[(16 * cc + 4 * gq + st) * AS + 16 * bb + m],
                                                   X, 0, 0, 0);
      }
      const floatx4 tv = *reinterpret_cast<const floatx4*>(&T32[(16 * a + m) * AS + 16 * a + 4 * gq]);
      floatx4 Y = zero;
#pragma unroll
      for (int st = 0; st < 4; ++st) Y = __builtin_amdgcn_mfma_f32_16x16x4f32(tv[st], X[st], Y, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) T32[(16 * a + 4 * gq + i) * AS + 16 * bb + m] = -Y[i];
    }
    __syncthreads();
  }
  // ---- P = Aqk M as P^T = M^T Aqk^T (so that each lane ends with its own row of P), split
  //      fp16 hi + lo. M = T diag(beta) is lower triangular: entries of tile blocks right of the
  //      diagonal (never written) are taken as zero.
  half8 pfh[2], pfl[2];
  if constexpr (!FACT) {
    floatx4 pt[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      pt[ct] = zero;
      if (ct > w) continue;  // P is lower triangular
      const float bj = Bs[16 * ct + m];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        half8 mt;  // M^T fragment: row 16ct + m of M^T = column of M, rows 32ks + kslot(gq, i)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int x = 32 * ks + kslot(gq, i);
          mt[i] = static_cast<_Float16>((x >> 4) >= ct ? T32[x * AS + 16 * ct + m] * bj : 0.f);
        }
        pt[ct] = mfma_f16(mt, ahi[ks], pt[ct]);
        pt[ct] = mfma_f16(mt, alo[ks], pt[ct]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        _Float16 hh, ll;
        split_f16(pt[2 * ks + (i >> 2)][i & 3], hh, ll);
        pfh[ks][i] = hh;
        pfl[ks][i] = ll;
      }
  }
  // ---- V fragments into the front of the arena (A is dead, T stays)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    half8 v16;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      v16[i] = static_cast<_Float16>(bf16_bits_to_f32(vraw[ks][i >> 2][i & 3]));
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      store_half_lds(reinterpret_cast<uint8_t*>(VBF), 2 * ks + hf, mfma_f16(v16, idf[hf], zero));
  }
  __syncthreads();
  if constexpr (FACT) {
    // ---- the factored block: Qbar and Aqk of row tile w as they are, Ktil^T fragments of key
    //      tiles 2w and 2w + 1, e^{G_C}, and for the column tiles 2w, 2w + 1 of every chunk row
    //      Utilde = M V (fp32 result tiles) and W = M Kbar computed transposed,
    //      W^T = Kbar^T M^T, so that each lane holds four keys of one token: half of an
    //      A-operand fragment of W (the other half is the other column tile).
    constexpr FLayout FL = flayout();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      *reinterpret_cast<half8*>(blk + FL.qb + ((kk * 4 + w) * 64 + l) * 16) = qbar[kk];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      *reinterpret_cast<half8*>(blk + FL.ah + ((ks * 4 + w) * 64 + l) * 16) = ahi[ks];
      *reinterpret_cast<half8*>(blk + FL.al + ((ks * 4 + w) * 64 + l) * 16) = alo[ks];
    }
#pragma unroll
    for (int f = 4 * w; f < 4 * w + 4; ++f)  // fragment f: key tile f / 2, token k-step f % 2
      *reinterpret_cast<half8*>(blk + FL.kt + (f * 64 + l) * 16) = KTL[f * 64 + l];
    if (t < DK) reinterpret_cast<float*>(blk + FL.gam)[t] = GAMS[t];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      half8 mr[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int bb = 2 * kk + hf;
          const floatx4 tv = *reinterpret_cast<const floatx4*>(&T32[(16 * rt + m) * AS + 16 * bb + 4 * gq]);
          const floatx4 bv = *reinterpret_cast<const floatx4*>(&Bs[16 * bb + 4 * gq]);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            mr[kk][4 * hf + ii] = static_cast<_Float16>(bb <= rt ? tv[ii] * bv[ii] : 0.f);
        }
      half8 wf;
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) {
        const int ct = 2 * w + tc;
        floatx4 dw = zero, du = zero;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          dw = mfma_f16(KBF[(ct * 2 + kk) * 64 + l], mr[kk], dw);
          du = mfma_f16(mr[kk], VBF[(ct * 2 + kk) * 64 + l], du);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) wf[4 * tc + i] = static_cast<_Float16>(dw[i]);
        *reinterpret_cast<floatx4*>(blk + FL.ut + ((ct * 4 + rt) * 64 + l) * 16) = du;
      }
      *reinterpret_cast<half8*>(blk + FL.w + ((rt * 4 + w) * 64 + l) * 16) = wf;
    }
    return;
  }
  // ---- row tile w: (P Kbar)^T = Kbar^T P^T, so that Qhat = Qbar - P Kbar comes out as
  //      A-operand fragments, and Ohat = P V as result tiles in the walk's accumulator layout.
  //      The second chunk of a composed block keeps both in registers for the composition.
  constexpr int RTB = BL / 16;  // row tiles of a block
  const bool second = COMPOSE && grp == 1;
  floatx4 ohb[8];  // second chunk: Ohat of row tile w, value tiles 0..7
  half8 qhb[4];    // second chunk: Qhat fragments of row tile w, k-steps 0..3
  // P's low fp16 part serves Ohat only: Qhat is stored in fp16, and P's high part alone leaves
  // its rounding unchanged (an emulation of every operand rounding of this path against the
  // oracle gives the same output error either way, while Ohat without it errs tenfold).
  floatx4 pk_prev = zero;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    floatx4 ap = zero, ao = zero;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const half8 kb = KBF[(ct * 2 + kk) * 64 + l];
      const half8 vb = VBF[(ct * 2 + kk) * 64 + l];
      ap = mfma_f16(kb, pfh[kk], ap);
      ao = mfma_f16(pfh[kk], vb, ao);
      ao = mfma_f16(pfl[kk], vb, ao);
    }
    if (second)
      ohb[ct] = ao;
    else
      *reinterpret_cast<floatx4*>(blk + LY.oh + (ct * RTB + w) * 1024 + l * 16) = ao;
    if (ct & 1) {  // tiles 2kk and 2kk + 1 form the fragments of k-step kk over dk
      const int kk = ct >> 1;
      half8 qh;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        qh[i] = static_cast<_Float16>(static_cast<float>(qbar[kk][i]) - (i < 4 ? pk_prev[i] : ap[i - 4]));
      if (second)
        qhb[kk] = qh;
      else
        *reinterpret_cast<half8*>(blk + LY.qh + (kk * RTB + w) * 1024 + l * 16) = qh;
    }
    pk_prev = ap;
  }
  // ---- W = M Kbar and Utilde = M V for the column tiles 2w and 2w + 1, every chunk row, as
  //      B-operand fragments [tile][k-step over chunk rows]: the result tile of row tile rt holds
  //      rows 16 rt + 4 gq + i of column m, i.e. half of the fragment of k-step rt / 2. M's row
  //      tiles come from T in LDS; Utilde is split fp16 hi + lo.
  half8 wb[2][2], uh[2][2], ul[2][2];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    half8 mr[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int bb = 2 * kk + hf;
        const floatx4 tv = *reinterpret_cast<const floatx4*>(&T32[(16 * rt + m) * AS + 16 * bb + 4 * gq]);
        const floatx4 bv = *reinterpret_cast<const floatx4*>(&Bs[16 * bb + 4 * gq]);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          mr[kk][4 * hf + ii] = static_cast<_Float16>(bb <= rt ? tv[ii] * bv[ii] : 0.f);
      }
#pragma unroll
    for (int tc = 0; tc < 2; ++tc) {
      const int ct = 2 * w + tc;
      floatx4 dw = zero, du = zero;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        dw = mfma_f16(mr[kk], KBF[(ct * 2 + kk) * 64 + l], dw);
        du = mfma_f16(mr[kk], VBF[(ct * 2 + kk) * 64 + l], du);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int slot = 4 * (rt & 1) + i;
        wb[tc][rt >> 1][slot] = static_cast<_Float16>(dw[i]);
        _Float16 hh, ll;
        split_f16(du[i], hh, ll);
        uh[tc][rt >> 1][slot] = hh;
        ul[tc][rt >> 1][slot] = ll;
      }
    }
  }
  // ---- composing a block: the two chunks hand each other their parts through staging areas
  //      in the parts of the arenas that only the products above read (V, M and Kbar^T;
  //      Ktil^T, still needed for Z, lies above them):
  //        PB  Psi of the second chunk, row fragments [key row tile][k-step]    arena 1 + 17408
  //        QB  Qhat of the second chunk, fragments [k-step][row tile]             arena 1 + 0
  //        ZA  Z of the first chunk, B-operand fragments [value tile][key pair]   arena 0 + 0
  half8* const PB = reinterpret_cast<half8*>(arenas[NGRP - 1] + 17408);
  half8* const QB = reinterpret_cast<half8*>(arenas[NGRP - 1]);
  half8* const ZA = reinterpret_cast<half8*>(arenas[0]);
  static_assert(17408 + 32768 <= OFF_KTL && 16384 <= 17408 && 32768 <= OFF_KTL, "staging");
  if constexpr (COMPOSE) {
    __syncthreads();  // every wave is past its last read of V, M and Kbar^T
    if (second) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) QB[(kk * 4 + w) * 64 + l] = qhb[kk];
    }
  }
  // ---- Phi = Ktil^T W for key rows kt and key columns 32w .. 32w + 31, computed as
  //      Phi^T = W^T Ktil so that each lane ends with its own row: A-operand fragments (kt, w).
  //      The first chunk of a composed block also forms Phi itself, whose result tiles are
  //      column fragments (a lane holds four rows of one column): the composition's A operand.
  half8 pra[8];     // first chunk: Psi row fragments (kt, w)
  half8 pca[2][4];  // first chunk: Psi column fragments (column tile 2w + tc, k-step over rows)
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    floatx4 d0 = zero, d1 = zero;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const half8 ktf = KTL[(kt * 2 + kk) * 64 + l];
      d0 = mfma_f16(wb[0][kk], ktf, d0);
      d1 = mfma_f16(wb[1][kk], ktf, d1);
    }
    // Psi = -Phi - Diag(1 - e^{G_C}): the diagonal entry of row 16 kt + m sits in k-step
    // kt / 2, in the lanes with gq = m / 4, slot (m mod 4) + 4 (kt mod 2)
    const int dslot = (kt >> 1) == w && gq == (m >> 2) ? (m & 3) + 4 * (kt & 1) : -1;
    const float dlt = dslot >= 0 ? 1.f - GAMS[16 * kt + m] : 0.f;
    half8 ph;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ph[i] = static_cast<_Float16>(-d0[i] - (i == dslot ? dlt : 0.f));
      ph[i + 4] = static_cast<_Float16>(-d1[i] - (i + 4 == dslot ? dlt : 0.f));
    }
    if (!COMPOSE)
      *reinterpret_cast<half8*>(blk + LY.phi + (kt * 4 + w) * 1024 + l * 16) = ph;
    else if (second)
      PB[(kt * 4 + w) * 64 + l] = ph;
    else
      pra[kt] = ph;
    if (COMPOSE && !second) {
      // tile (kt, 2w + tc) of Phi: the lane holds column 16 (2w + tc) + m, rows 16 kt + 4 gq + i,
      // the diagonal where 16 kt + 4 gq + i = 16 (2w + tc) + m
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) {
        floatx4 e = zero;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) e = mfma_f16(KTL[(kt * 2 + kk) * 64 + l], wb[tc][kk], e);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool diag = kt == 2 * w + tc && 4 * gq + i == m;
          pca[tc][kt >> 1][4 * (kt & 1) + i] =
              static_cast<_Float16>(-e[i] - (diag ? 1.f - GAMS[16 * kt + m] : 0.f));
        }
      }
    }
  }
  // ---- Z = Ktil^T Utilde for value tiles 2w and 2w + 1, every key row tile: the lane holds
  //      key rows 16 kt + 4 gq + i of value column m, the walk's accumulator layout (fp16).
  //      Composing: the first chunk's Z goes to ZA, the second chunk's stays in fp32 registers.
  floatx4 zb[2][8];  // second chunk: Z tiles (value tile 2w + tt, key row tile kt)
#pragma unroll
  for (int kp = 0; kp < 4; ++kp)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      half8 zf;  // key row tiles 2kp and 2kp + 1: one 16-byte store
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int kt = 2 * kp + u;
        const half8 kf0 = KTL[(kt * 2) * 64 + l], kf1 = KTL[(kt * 2 + 1) * 64 + l];
        floatx4 dz = zero, dz2 = zero;
        dz = mfma_f16(kf0, uh[tt][0], dz);
        dz2 = mfma_f16(kf0, ul[tt][0], dz2);
        dz = mfma_f16(kf1, uh[tt][1], dz);
        dz2 = mfma_f16(kf1, ul[tt][1], dz2);
        if (second) zb[tt][kt] = dz + dz2;
#pragma unroll
        for (int i = 0; i < 4; ++i) zf[4 * u + i] = static_cast<_Float16>(dz[i] + dz2[i]);
      }
      const int vt = 2 * w + tt;
      if (!COMPOSE)
        *reinterpret_cast<half8*>(blk + LY.z + ((vt * 4 + kp) * 64 + l) * 16) = zf;
      else if (!second)
        ZA[(vt * 4 + kp) * 64 + l] = zf;
    }
  if constexpr (COMPOSE) {
    // ---- the block's step from the two chunks' steps S -> S + Z + Psi S:
    //        Psi'    = Psi_a + Psi_b + Psi_b Psi_a
    //        Z'      = Z_a + Z_b + Psi_b Z_a
    //        Qhat'_b = Qhat_b + Qhat_b Psi_a,   Ohat'_b = Ohat_b + Qhat_b Z_a
    //      (the second chunk's outputs read the state entering the block); the first chunk's
    //      Qhat and Ohat are stored as they are.
    __syncthreads();  // PB, QB and ZA are complete
    if (!second) {
      // Psi' row fragments (kt, w) as the transposed product Psi_a^T Psi_b^T: each lane ends
      // with four entries of its own row of Psi' per 16-column tile 2w + tc
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        half8 pb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) pb[ks] = PB[(kt * 4 + ks) * 64 + l];
        const half8 pbw = w == 0 ? pb[0] : w == 1 ? pb[1] : w == 2 ? pb[2] : pb[3];  // seed (kt, w)
        floatx4 acc[2];
#pragma unroll
        for (int tc = 0; tc < 2; ++tc)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[tc][i] = static_cast<float>(pra[kt][4 * tc + i]) + static_cast<float>(pbw[4 * tc + i]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int tc = 0; tc < 2; ++tc) acc[tc] = mfma_f16(pca[tc][ks], pb[ks], acc[tc]);
        half8 out;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          out[i] = static_cast<_Float16>(acc[0][i]);
          out[i + 4] = static_cast<_Float16>(acc[1][i]);
        }
        *reinterpret_cast<half8*>(blk + LY.phi + (kt * 4 + w) * 1024 + l * 16) = out;
      }
      // Qhat'_b fragments (k-step w, row tile rt of the second chunk), transposed likewise
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        half8 qb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qb[ks] = QB[(ks * 4 + rt) * 64 + l];
        const half8 qbw = w == 0 ? qb[0] : w == 1 ? qb[1] : w == 2 ? qb[2] : qb[3];  // seed (w, rt)
        floatx4 acc[2];
#pragma unroll
        for (int tc = 0; tc < 2; ++tc)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[tc][i] = static_cast<float>(qbw[4 * tc + i]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int tc = 0; tc < 2; ++tc) acc[tc] = mfma_f16(pca[tc][ks], qb[ks], acc[tc]);
        half8 out;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          out[i] = static_cast<_Float16>(acc[0][i]);
          out[i + 4] = static_cast<_Float16>(acc[1][i]);
        }
        *reinterpret_cast<half8*>(blk + LY.qh + (w * RTB + 4 + rt) * 1024 + l * 16) = out;
      }
    } else {
      // Z' tiles (key row tile r, value tile 2w + tt), in the walk's layout. Z_a's fragments
      // of this wave's two value tiles stay in registers; each Psi_b fragment is read once.
      half8 za[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) za[tt][ks] = ZA[((2 * w + tt) * 4 + ks) * 64 + l];
#pragma unroll
      for (int kp = 0; kp < 4; ++kp) {
        half8 zo[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 2 * kp + u;
          half8 pb[4];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) pb[ks] = PB[(r * 4 + ks) * 64 + l];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            floatx4 acc = zb[tt][r];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += static_cast<float>(za[tt][kp][4 * u + i]);  // Z_a
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) acc = mfma_f16(pb[ks], za[tt][ks], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) zo[tt][4 * u + i] = static_cast<_Float16>(acc[i]);
          }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          *reinterpret_cast<half8*>(blk + LY.z + (((2 * w + tt) * 4 + kp) * 64 + l) * 16) = zo[tt];
      }
      // Ohat'_b tiles (value tile vt, row tile w of the second chunk)
#pragma unroll
      for (int vt = 0; vt < 8; ++vt) {
        floatx4 acc = ohb[vt];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bool mine = (vt >> 1) == w;  // already in registers
          acc = mfma_f16(qhb[ks], mine ? za[vt & 1][ks] : ZA[(vt * 4 + ks) * 64 + l], acc);
        }
        *reinterpret_cast<floatx4*>(blk + LY.oh + (vt * RTB + 4 + w) * 1024 + l * 16) = acc;
      }
    }
  }
}

// ---------------------------------------------------------------- rec
__device__ __forceinline__ half8 ld_frag(rsrc_t r, int lane_off, int off) {
  return __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, off, 0));
}
__device__ __forceinline__ floatx4 ld_tile(rsrc_t r, int lane_off, int off) {
  return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, off, 0));
}

// One walk of the recurrence over chunks c_lo .. c_hi - 1 of every sequence (those that exist;
// chunk indices, and with them the workspace blocks, checkpoints and outputs, are the
// sequence's own), for every (sequence, head):
//   REC_OUTPUT      from S_in (zeros if null): outputs and checkpoints written;
//   REC_SUMMARY     from zeros, nothing but the exit state: the segment's zero-start summary Z;
//   REC_TRANSITION  from the identity with V = 0 (Utilde = 0), nothing but the exit state:
//                   the segment's transition Phi, so that S_exit = Phi S_entry + Z.
// The exit state goes to S_out when it is not null.
enum { REC_OUTPUT = 0, REC_SUMMARY = 1, REC_TRANSITION = 2 };
struct RecJob {
  int64_t c_lo, c_hi;
  const float* S_in;
  float* S_out;
  int mode;
};
constexpr int kMaxJobs = 16;
struct RecJobs {
  RecJob job[kMaxJobs];
  int64_t blocks_per_job;
  int halves;  // 2: two workgroups per strip run the same state walk, each with the outputs of
               // half of the chunk rows (fewer operand bytes per CU when CUs would be idle)
};

template <int N>
struct IntC {
  static constexpr int value = N;
};

// The walk steps over workspace blocks of BL tokens (one chunk of 64, or two composed into
// 128); below, "chunk" c is such a block. CKPT: the launch stores state checkpoints (a kernel
// of its own, so that the plain walk's loop holds no conditional stores: the compiler would
// otherwise drain every load in flight at their merge, once per unrolled loop trip).
template <typename TOut, int NT, int BL, bool CKPT>
__global__ __launch_bounds__(512) void rec_kernel(
    RecJobs jobs, TOut* __restrict__ o, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_off, int T, int H, int n_seq, int64_t max_chunks,
    const uint8_t* __restrict__ ws, float* __restrict__ ckpt, int ckpt_chunks, int ckpt_slots,
    const int32_t* __restrict__ ckpt_off, const int32_t* __restrict__ order) {
  // blockIdx.x = job * blocks_per_job + (block within the job)
  // A workgroup owns NT strips of 16 value columns. One fp16 exchange per chunk through LDS,
  // followed by one barrier: the state strips entering the chunk (all 128 key rows), which the
  // state waves need whole for Psi S and the output waves for Qhat S. They are stored
  // column-major ([column][row]) so the rows a lane needs for a B operand are contiguous, with
  // rows padded by 4 halves (the fragment reads of 16 lanes then fall into distinct banks; 8
  // halves measured 2-way bank conflicts), in two buffers used by alternate chunks:
  // the buffer of chunk c is read between barrier c and barrier c + 1, and written again only
  // for chunk c + 2, after barrier c + 1.
  constexpr Layout LY = layout(BL);
  constexpr int RT = BL / 16;      // row tiles of a chunk
  constexpr int NG = NSTRIP / NT;  // strip groups per (sequence, head)
  constexpr int SR = DK + 4;  // 66 words per row: conflict-free fragment reads
  __shared__ __align__(16) _Float16 sx[2][NT * 16][SR];

  const RecJob job = jobs.job[blockIdx.x / jobs.blocks_per_job];
  const int64_t c_lo = job.c_lo, c_hi = job.c_hi;
  const float* __restrict__ S0 = job.mode == REC_OUTPUT ? job.S_in : nullptr;
  float* __restrict__ S_T = job.S_out;
  const bool transition = job.mode == REC_TRANSITION;
  // XCD-aware placement: the strip groups of one (sequence, head) share an XCD and its L2.
  const int b = (int)(blockIdx.x % jobs.blocks_per_job);
  const int xcd = b & 7, rest = b >> 3;
  const int sg = rest % NG, r2 = rest / NG;
  const int half = r2 % jobs.halves;
  const int64_t pair = (int64_t)(r2 / jobs.halves) * 8 + xcd;
  if (pair >= (int64_t)n_seq * H) return;
  // packed sequences are walked longest first (order from the plan kernel)
  const int n = order ? order[pair / H] : (int)(pair / H), h = (int)(pair % H);
  const SeqInfo si = seq_info<BL>(n, cu, chunk_off, T);
  // a malformed cu_seqlens cannot make the chunk walk leave the workspace
  const int64_t nc = max((int64_t)0, min((si.len + BL - 1) / BL, max_chunks - si.cid0));
  const int64_t c_end = min(nc, c_hi);  // this launch walks chunks c_lo .. c_end - 1

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int w = wave & 3;
  const int l = t & 63, gq = l >> 4, nn = l & 15;
  const int frag_off = l * 16;
  const uint8_t* blk_base = ws + ((size_t)si.cid0 * H + h) * LY.block;
  const size_t blk_step = (size_t)H * LY.block;

  // B operand of state strip nt for key rows 32 j + kslot(gq, i), column nn, from buffer bf
  auto state_frag = [&](int bf, int nt, int j) { return lds_frag(&sx[bf][16 * nt + nn][32 * j], gq); };
  // first checkpoint slot of this sequence (checkpoints every ckpt_chunks full chunks)
  const int64_t ck_base =
      ckpt_chunks > 0 ? (cu ? (int64_t)ckpt_off[n] : (int64_t)n * (T / (ckpt_chunks * BL))) : 0;
  // the second workgroup of a split pair repeats the walk: only the first writes states. Both
  // read S0 when they start, so the split assumes S0 is not written during the launch (the
  // host never splits an in-place walk, where S_T is the S0 buffer).
  const int ck_every = CKPT && job.mode == REC_OUTPUT && half == 0 ? ckpt_chunks : 0;
  if (half != 0) S_T = nullptr;

  // ------------------------------------------------ output waves: chunk rows of JN row tiles
  // (rt0, and rt1 when JN = 2), o = Qhat S + Ohat from the state entering the chunk. The tile
  // count is a compile-time constant, so that the loop holds no branch around its loads and
  // the compiler keeps its waits partial (two chunks of operands in flight).
  auto out_waves = [&](auto jn, int rt0, int rt1) {
    constexpr int JN = decltype(jn)::value;
    const int rts[2] = {rt0, rt1};
    const int row_stride = H * DV;  // elements between consecutive tokens
    int o_off[JN][NT][4];
#pragma unroll
    for (int j = 0; j < JN; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o_off[j][nt][i] = ((16 * rts[j] + 4 * gq + i) * row_stride + 16 * (NT * sg + nt) + nn) *
                            (int)sizeof(TOut);
    TOut* o_base = o + (si.tok0 * H + h) * DV;
    const size_t tok_step = (size_t)BL * row_stride;
    struct Ops {
      half8 qh[JN][4];
      floatx4 oh[JN][NT];
    };
    Ops A, B;
    auto load_q = [&](Ops& X, int64_t c) {
      const rsrc_t r = make_rsrc(blk_base + min(c, c_end - 1) * blk_step, (int64_t)LY.block);
#pragma unroll
      for (int j = 0; j < JN; ++j) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) X.qh[j][ks] = ld_frag(r, frag_off, LY.qh + (ks * RT + rts[j]) * 1024);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          X.oh[j][nt] = ld_tile(r, frag_off, LY.oh + ((NT * sg + nt) * RT + rts[j]) * 1024);
      }
    };
    auto step = [&](Ops& X, int64_t c) {
      const int bf = (int)(c & 1);
      __syncthreads();
      // the products read the state entering the chunk, from the buffer the state waves
      // filled before this barrier
      floatx4 acc[JN][NT];
#pragma unroll
      for (int j = 0; j < JN; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          floatx4 a0 = mfma_f16(X.qh[j][0], state_frag(bf, nt, 0), X.oh[j][nt]);
          floatx4 a1 = mfma_f16(X.qh[j][2], state_frag(bf, nt, 2), floatx4{0.f, 0.f, 0.f, 0.f});
          a0 = mfma_f16(X.qh[j][1], state_frag(bf, nt, 1), a0);
          a1 = mfma_f16(X.qh[j][3], state_frag(bf, nt, 3), a1);
          acc[j][nt] = a0 + a1;
        }
      load_q(X, c + 2);
      // bytes of the chunk's rows of this head, up to the end of its last valid row
      const int64_t rows = min((int64_t)BL, si.len - c * BL);
      const rsrc_t ro = make_rsrc(o_base + c * tok_step, ((rows - 1) * row_stride + DV) * (int64_t)sizeof(TOut));
#pragma unroll
      for (int j = 0; j < JN; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (sizeof(TOut) == 4)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[j][nt][i]), ro, o_off[j][nt][i], 0, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(acc[j][nt][i]), ro, o_off[j][nt][i], 0, 0);
          }
    };
    if (c_end > c_lo) {
      load_q(A, c_lo);
      load_q(B, c_lo + 1);
    }
    __builtin_amdgcn_s_waitcnt(0);  // as for the state waves: the loop waits stay partial
    int64_t c = c_lo;
    for (; c + 1 < c_end; c += 2) {
      step(A, c);
      step(B, c + 1);
    }
    if (c < c_end) step(A, c);
  };

  if (wave < 4) {
    // ------------------------------------------------ state waves: key rows 32w .. 32w+31
    // they carry the serial chain: when both roles have work ready on a SIMD, theirs issues first
    __builtin_amdgcn_s_setprio(2);
    const int64_t s_base = ((int64_t)n * H + h) * DK * DV;
    int col[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) col[nt] = 16 * (NT * sg + nt) + nn;
    // rows 32w + 16u + 4gq + i (u = 0, 1), columns col[nt]
    floatx4 s[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 32 * w + 16 * u + 4 * gq + i;
          s[nt][u][i] = transition ? (r == col[nt] ? 1.f : 0.f)
                                   : (S0 ? S0[s_base + (int64_t)r * DV + col[nt]] : 0.f);
        }

    // Operands are loaded two chunks ahead into three register sets used in rotation (the
    // loop is unrolled by three, so no set is ever copied): a chunk's loads have two chunks'
    // time to arrive, which covers a first read of the workspace from HBM, and the set being
    // filled is idle for the whole step, so its loads are spread over the step in three
    // groups instead of leaving the vector memory unit one burst to drain while the chain
    // waits behind it.
    struct Ops {
      half8 phi[2][4];  // Psi rows of key row tiles 2w + u, k-steps over keys
      half8 z[NT];      // Z of both key row tiles for strip nt (fp16, accumulator layout)
    };
    Ops A, B, Cs;
    auto load_part = [&](Ops& X, rsrc_t r, int part) {
      if (part < 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) X.phi[part][j] = ld_frag(r, frag_off, LY.phi + ((2 * w + part) * 4 + j) * 1024);
      } else {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) X.z[nt] = ld_frag(r, frag_off, LY.z + ((NT * sg + nt) * 4 + w) * 1024);
      }
    };
    auto load_ops = [&](Ops& X, rsrc_t r) {
      load_part(X, r, 2);
      load_part(X, r, 0);
      load_part(X, r, 1);
    };
    auto chunk_rsrc = [&](int64_t c) {
      return make_rsrc(blk_base + min(c, c_end - 1) * blk_step, (int64_t)LY.block);
    };
    // one chunk with operand set X, while set Y (idle since the previous chunk) is loaded with
    // chunk c + 2 (past the end, the last chunk reloads itself), unconditionally and in a
    // fixed order, so the loop has no branch
    auto step = [&](Ops& X, Ops& Y, int64_t c) {
      const rsrc_t rn = chunk_rsrc(c + 2);
      const int bf = (int)(c & 1);
      // S + Z seeds the accumulators, off the chain (the transition walk has V = 0, so Z = 0)
      floatx4 seed[NT][2];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            seed[nt][u][i] = s[nt][u][i] + (transition ? 0.f : static_cast<float>(X.z[nt][4 * u + i]));
      // -- all-gather the state strips in fp16
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          half4 hv;
#pragma unroll
          for (int i = 0; i < 4; ++i) hv[i] = static_cast<_Float16>(s[nt][u][i]);
          *reinterpret_cast<half4*>(&sx[bf][16 * nt + nn][32 * w + 16 * u + 4 * gq]) = hv;
        }
      load_part(Y, rn, 2);  // Z first: the next use of a set begins with its Z (the seed)
      load_part(Y, rn, 0);
      __syncthreads();
      // -- this wave's state rows: S = S + Z + Psi S, where Psi S runs as four
      //    independent accumulation chains (two row tiles, two halves of the key range)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        half8 sf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sf[j] = state_frag(bf, nt, j);
        if (nt == 0) load_part(Y, rn, 1);
        floatx4 a0[2], a1[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          a0[u] = mfma_f16(X.phi[u][0], sf[0], seed[nt][u]);
          a1[u] = mfma_f16(X.phi[u][2], sf[2], floatx4{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          a0[u] = mfma_f16(X.phi[u][1], sf[1], a0[u]);
          a1[u] = mfma_f16(X.phi[u][3], sf[3], a1[u]);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) s[nt][u] = a0[u] + a1[u];
      }
      // -- the state after every ckpt_chunks full chunks, if asked for
      if (CKPT && ck_every > 0 && (c + 1) % ck_every == 0 && (c + 1) * BL <= si.len) {
        const int64_t slot = ck_base + (c + 1) / ck_every - 1;
        if (slot < ckpt_slots) {
          float* dst = ckpt + (slot * H + h) * DK * DV;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int i = 0; i < 4; ++i) dst[(int64_t)(32 * w + 16 * u + 4 * gq + i) * DV + col[nt]] = s[nt][u][i];
        }
      }
    };
    if (c_end > c_lo) {
      load_ops(A, chunk_rsrc(c_lo));
      load_ops(B, chunk_rsrc(c_lo + 1));
    }
    // Nothing may be pending on entry to the loop: the compiler computes the loop's memory
    // waits from the merge of its entry paths and the back edge, and loads left in flight on
    // an entry path (the conditional ones above) would turn every wait in the loop into a
    // full one.
    __builtin_amdgcn_s_waitcnt(0);
    int64_t c = c_lo;
    for (; c + 2 < c_end; c += 3) {
      step(A, Cs, c);
      step(B, A, c + 1);
      step(Cs, B, c + 2);
    }
    if (c < c_end) step(A, Cs, c);
    if (c + 1 < c_end) step(B, A, c + 1);
    if (S_T) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            S_T[s_base + (int64_t)(32 * w + 16 * u + 4 * gq + i) * DV + col[nt]] = s[nt][u][i];
    }
  } else if (job.mode != REC_OUTPUT || (RT == 4 && jobs.halves == 2 && (w >> 1) != half)) {
    // ------------------------------------------------ no outputs: keep the barriers in step
    for (int64_t c = c_lo; c < c_end; ++c) __syncthreads();
  } else if (RT == 8 && jobs.halves == 1) {
    out_waves(IntC<2>{}, w, w + 4);   // every output wave: row tiles w and w + 4
  } else {
    // one row tile per output wave: tile w (RT = 4, or RT = 8 with each workgroup of a split
    // pair taking the first or the last four row tiles)
    out_waves(IntC<1>{}, RT == 8 ? w + 4 * half : w, 0);
  }
}

// The walk over factored blocks (one 64-token chunk per step). Per chunk, with S the state
// entering it:
//   U' = Utilde - W S,   o = Qbar S + Aqk U',   S <- Diag(e^{G_C}) S + Ktil^T U'.
// State wave w holds key rows 32w .. 32w+31 of the strips. Its own rows, converted to fp16,
// are exactly the B operand of k-step w, so it forms its part of W S over those keys without
// any exchange: X_w = W[:, 32w..32w+31] S[32w..32w+31, :], four result tiles (one per token
// row tile). The four parts meet in LDS; wave w adds them for token tile w and forms
// U' = Utilde - X there (fp16 high and low parts); after a second barrier every wave reads
// the whole U' as B operands for Ktil^T U' (its key rows) and for Aqk U' (the output waves,
// with high and low parts of both). The output waves read the state entering the chunk, as
// in rec_kernel, for Qbar S.
template <typename TOut, int NT, bool CKPT>
__global__ __launch_bounds__(512) void rec_fact_kernel(
    RecJobs jobs, TOut* __restrict__ o, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_off, int T, int H, int n_seq, int64_t max_chunks,
    const uint8_t* __restrict__ ws, float* __restrict__ ckpt, int ckpt_chunks, int ckpt_slots,
    const int32_t* __restrict__ ckpt_off, const int32_t* __restrict__ order) {
  constexpr FLayout FL = flayout();
  constexpr int BL = C;
  constexpr int NG = NSTRIP / NT;
  constexpr int SR = DK + 4;  // 66 words per row: conflict-free fragment reads
  __shared__ __align__(16) _Float16 sx[2][NT * 16][SR];  // state entering the chunk, fp16
  __shared__ __align__(16) floatx4 xp[4][NT][4][64];     // parts of W S [wave][strip][token tile]
  __shared__ __align__(16) half4 up[NT][4][2][64];       // U' [strip][token tile][high, low]

  const RecJob job = jobs.job[blockIdx.x / jobs.blocks_per_job];
  const int64_t c_lo = job.c_lo, c_hi = job.c_hi;
  const float* __restrict__ S0 = job.mode == REC_OUTPUT ? job.S_in : nullptr;
  float* __restrict__ S_T = job.S_out;
  const bool transition = job.mode == REC_TRANSITION;
  const int b = (int)(blockIdx.x % jobs.blocks_per_job);
  const int xcd = b & 7, rest = b >> 3;
  const int sg = rest % NG, r2 = rest / NG;
  const int half = r2 % jobs.halves;
  const int64_t pair = (int64_t)(r2 / jobs.halves) * 8 + xcd;
  if (pair >= (int64_t)n_seq * H) return;
  const int n = order ? order[pair / H] : (int)(pair / H), h = (int)(pair % H);
  const SeqInfo si = seq_info<BL>(n, cu, chunk_off, T);
  const int64_t nc = max((int64_t)0, min((si.len + BL - 1) / BL, max_chunks - si.cid0));
  const int64_t c_end = min(nc, c_hi);

  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int w = wave & 3;
  const int l = t & 63, gq = l >> 4, nn = l & 15;
  const int frag_off = l * 16;
  const uint8_t* blk_base = ws + ((size_t)si.cid0 * H + h) * FL.block;
  const size_t blk_step = (size_t)H * FL.block;
  auto chunk_rsrc = [&](int64_t c) {
    return make_rsrc(blk_base + min(c, c_end - 1) * blk_step, (int64_t)FL.block);
  };
  auto state_frag = [&](int bf, int nt, int j) { return lds_frag(&sx[bf][16 * nt + nn][32 * j], gq); };
  // U' high (hl = 0) or low (1) parts as the B operand of token k-step jt: token tiles 2jt and
  // 2jt + 1, the lane's own four rows of each
  auto u_frag = [&](int nt, int jt, int hl) {
    return frag_from_halves(up[nt][2 * jt][hl][l], up[nt][2 * jt + 1][hl][l]);
  };
  const int64_t ck_base =
      ckpt_chunks > 0 ? (cu ? (int64_t)ckpt_off[n] : (int64_t)n * (T / (ckpt_chunks * BL))) : 0;
  const int ck_every = CKPT && job.mode == REC_OUTPUT && half == 0 ? ckpt_chunks : 0;
  if (half != 0) S_T = nullptr;

  // ------------------------------------------------ output waves: chunk rows of JN row tiles
  auto out_waves = [&](auto jn, int rt0, int rt1) {
    constexpr int JN = decltype(jn)::value;
    const int rts[2] = {rt0, rt1};
    const int row_stride = H * DV;
    int o_off[JN][NT][4];
#pragma unroll
    for (int j = 0; j < JN; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o_off[j][nt][i] = ((16 * rts[j] + 4 * gq + i) * row_stride + 16 * (NT * sg + nt) + nn) *
                            (int)sizeof(TOut);
    TOut* o_base = o + (si.tok0 * H + h) * DV;
    const size_t tok_step = (size_t)BL * row_stride;
    struct Ops {
      half8 qb[JN][4];  // Qbar, key k-steps
      half8 ah[JN][2], al[JN][2];  // Aqk high and low parts, token k-steps
    };
    Ops A, B;
    auto load_q = [&](Ops& X, int64_t c) {
      const rsrc_t r = chunk_rsrc(c);
#pragma unroll
      for (int j = 0; j < JN; ++j) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) X.qb[j][ks] = ld_frag(r, frag_off, FL.qb + (ks * 4 + rts[j]) * 1024);
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
          X.ah[j][jt] = ld_frag(r, frag_off, FL.ah + (jt * 4 + rts[j]) * 1024);
          X.al[j][jt] = ld_frag(r, frag_off, FL.al + (jt * 4 + rts[j]) * 1024);
        }
      }
    };
    auto step = [&](Ops& X, int64_t c) {
      const int bf = (int)(c & 1);
      __syncthreads();  // A: the state entering chunk c is in sx[bf]
      // Qbar S while the state waves form U'
      floatx4 a0[JN][NT], a1[JN][NT];
#pragma unroll
      for (int j = 0; j < JN; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          a0[j][nt] = mfma_f16(X.qb[j][0], state_frag(bf, nt, 0), floatx4{0.f, 0.f, 0.f, 0.f});
          a1[j][nt] = mfma_f16(X.qb[j][2], state_frag(bf, nt, 2), floatx4{0.f, 0.f, 0.f, 0.f});
          a0[j][nt] = mfma_f16(X.qb[j][1], state_frag(bf, nt, 1), a0[j][nt]);
          a1[j][nt] = mfma_f16(X.qb[j][3], state_frag(bf, nt, 3), a1[j][nt]);
        }
      __syncthreads();  // B: U' of chunk c is in up
      floatx4 acc[JN][NT];
#pragma unroll
      for (int j = 0; j < JN; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            const half8 uh = u_frag(nt, jt, 0), ul = u_frag(nt, jt, 1);
            a0[j][nt] = mfma_f16(X.ah[j][jt], uh, a0[j][nt]);
            a1[j][nt] = mfma_f16(X.ah[j][jt], ul, a1[j][nt]);
            a1[j][nt] = mfma_f16(X.al[j][jt], uh, a1[j][nt]);
          }
          acc[j][nt] = a0[j][nt] + a1[j][nt];
        }
      load_q(X, c + 2);
      const int64_t rows = min((int64_t)BL, si.len - c * BL);
      const rsrc_t ro = make_rsrc(o_base + c * tok_step, ((rows - 1) * row_stride + DV) * (int64_t)sizeof(TOut));
#pragma unroll
      for (int j = 0; j < JN; ++j)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (sizeof(TOut) == 4)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[j][nt][i]), ro, o_off[j][nt][i], 0, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(acc[j][nt][i]), ro, o_off[j][nt][i], 0, 0);
          }
    };
    if (c_end > c_lo) {
      load_q(A, c_lo);
      load_q(B, c_lo + 1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    int64_t c = c_lo;
    for (; c + 1 < c_end; c += 2) {
      step(A, c);
      step(B, c + 1);
    }
    if (c < c_end) step(A, c);
  };

  if (wave < 4) {
    // ------------------------------------------------ state waves: key rows 32w .. 32w+31
    __builtin_amdgcn_s_setprio(2);
    const int64_t s_base = ((int64_t)n * H + h) * DK * DV;
    int col[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) col[nt] = 16 * (NT * sg + nt) + nn;
    floatx4 s[NT][2];  // rows 32w + 16u + 4gq + i, columns col[nt]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 32 * w + 16 * u + 4 * gq + i;
          s[nt][u][i] = transition ? (r == col[nt] ? 1.f : 0.f)
                                   : (S0 ? S0[s_base + (int64_t)r * DV + col[nt]] : 0.f);
        }
    // Operands two chunks ahead in three register sets used in rotation, as in rec_kernel.
    // The transition walk has V = 0: its Utilde loads read an empty range (zeros).
    const int ut_bytes = transition ? 0 : FL.block;
    struct Ops {
      half8 wf[4];     // W fragments of token tiles 0..3, key k-step w
      half8 kf[2][2];  // Ktil^T fragments of key tiles 2w + u, token k-steps jt
      floatx4 ut[NT];  // Utilde of token tile w, value tiles of the strips
      floatx4 gm[2];   // e^{G_C} of key rows 32w + 16u + 4gq .. + 3
    };
    Ops A, B, Cs;
    auto load_ops = [&](Ops& X, int64_t c) {
      const uint8_t* base = blk_base + min(c, c_end - 1) * blk_step;
      const rsrc_t r = make_rsrc(base, (int64_t)FL.block);
      const rsrc_t ru = make_rsrc(base, (int64_t)ut_bytes);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) X.ut[nt] = ld_tile(ru, frag_off, FL.ut + ((NT * sg + nt) * 4 + w) * 1024);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) X.wf[rt] = ld_frag(r, frag_off, FL.w + (rt * 4 + w) * 1024);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) X.kf[u][jt] = ld_frag(r, frag_off, FL.kt + ((2 * w + u) * 2 + jt) * 1024);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        X.gm[u] = ld_tile(r, (32 * w + 16 * u + 4 * gq) * 4, FL.gam);
    };
    auto step = [&](Ops& X, Ops& Y, int64_t c) {
      const int bf = (int)(c & 1);
      // -- the state entering the chunk: fp16 for the output waves, and this wave's own rows
      //    as the B operand of key k-step w
      half8 sw[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          half4 hv;
#pragma unroll
          for (int i = 0; i < 4; ++i) hv[i] = static_cast<_Float16>(s[nt][u][i]);
          *reinterpret_cast<half4*>(&sx[bf][16 * nt + nn][32 * w + 16 * u + 4 * gq]) = hv;
#pragma unroll
          for (int i = 0; i < 4; ++i) sw[nt][4 * u + i] = hv[i];
        }
      // -- this wave's part of W S, token tiles 0..3
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          xp[w][nt][rt][l] = mfma_f16(X.wf[rt], sw[nt], floatx4{0.f, 0.f, 0.f, 0.f});
      load_ops(Y, c + 2);
      __syncthreads();  // A
      // -- U' of token tile w: Utilde - (sum of the four parts), high and low fp16 parts
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const floatx4 x = (xp[0][nt][w][l] + xp[1][nt][w][l]) + (xp[2][nt][w][l] + xp[3][nt][w][l]);
        const floatx4 uu = X.ut[nt] - x;
        half4 hi, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hi[i] = static_cast<_Float16>(uu[i]);
          lo[i] = static_cast<_Float16>(uu[i] - static_cast<float>(hi[i]));
        }
        up[nt][w][0][l] = hi;
        up[nt][w][1][l] = lo;
      }
      __syncthreads();  // B
      // -- S <- Diag(e^{G_C}) S + Ktil^T U' for this wave's rows
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const half8 u0 = u_frag(nt, 0, 0), u1 = u_frag(nt, 1, 0);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          floatx4 seed;
#pragma unroll
          for (int i = 0; i < 4; ++i) seed[i] = s[nt][u][i] * X.gm[u][i];
          seed = mfma_f16(X.kf[u][0], u0, seed);
          s[nt][u] = mfma_f16(X.kf[u][1], u1, seed);
        }
      }
      if (CKPT && ck_every > 0 && (c + 1) % ck_every == 0 && (c + 1) * BL <= si.len) {
        const int64_t slot = ck_base + (c + 1) / ck_every - 1;
        if (slot < ckpt_slots) {
          float* dst = ckpt + (slot * H + h) * DK * DV;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int i = 0; i < 4; ++i) dst[(int64_t)(32 * w + 16 * u + 4 * gq + i) * DV + col[nt]] = s[nt][u][i];
        }
      }
    };
    if (c_end > c_lo) {
      load_ops(A, c_lo);
      load_ops(B, c_lo + 1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    int64_t c = c_lo;
    for (; c + 2 < c_end; c += 3) {
      step(A, Cs, c);
      step(B, A, c + 1);
      step(Cs, B, c + 2);
    }
    if (c < c_end) step(A, Cs, c);
    if (c + 1 < c_end) step(B, A, c + 1);
    if (S_T) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            S_T[s_base + (int64_t)(32 * w + 16 * u + 4 * gq + i) * DV + col[nt]] = s[nt][u][i];
    }
  } else if (job.mode != REC_OUTPUT || (jobs.halves == 2 && (w >> 1) != half)) {
    // ------------------------------------------------ no outputs: keep the barriers in step
    for (int64_t c = c_lo; c < c_end; ++c) {
      __syncthreads();
      __syncthreads();
    }
  } else {
    // one row tile per output wave: tile w (each workgroup of a split pair takes half of them)
    out_waves(IntC<1>{}, w, 0);
  }
}

// Entry state of the next segment from the previous one's: S_next = Phi S_in + Z, per
// (sequence, head), fp32. One workgroup per (sequence, head, 16-column strip); Phi is streamed
// through LDS in 32-column slabs.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ Phi,
                                                      const float* __restrict__ S_in,
                                                      const float* __restrict__ Z,
                                                      float* __restrict__ S_next, int64_t pairs) {
  const int64_t pair = blockIdx.x / NSTRIP;
  const int strip = blockIdx.x % NSTRIP;
  if (pair >= pairs) return;
  __shared__ float sin_s[DK][17];   // S_in strip, [key row][column]
  __shared__ float phi_s[DK][33];   // Phi rows, one 32-column slab at a time
  const int t = threadIdx.x;
  const int64_t base = pair * DK * DV;
  for (int i = t; i < DK * 16; i += 256)
    sin_s[i / 16][i % 16] = S_in[base + (int64_t)(i / 16) * DV + 16 * strip + i % 16];
  const int j = t & 15, r0 = (t >> 4) * 8;  // this thread: rows r0 .. r0 + 7 of column j
  float acc[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) acc[rr] = Z[base + (int64_t)(r0 + rr) * DV + 16 * strip + j];
  for (int kb = 0; kb < DK; kb += 32) {
    __syncthreads();
    for (int i = t; i < DK * 32; i += 256)
      phi_s[i / 32][i % 32] = Phi[base + (int64_t)(i / 32) * DK + kb + i % 32];
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      const float sv = sin_s[kb + kk][j];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) acc[rr] = fmaf(phi_s[r0 + rr][kk], sv, acc[rr]);
    }
  }
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) S_next[base + (int64_t)(r0 + rr) * DV + 16 * strip + j] = acc[rr];
}

// Tokens per workspace block and walk step (chosen with the plan): 64, one chunk, or 128, two
// chunks composed.
int walk_block(const ChunkPlan& p) { return p.walk_block == 2 * C ? 2 * C : C; }

int64_t max_blocks(const ChunkPlan& p) {
  const int BL = walk_block(p);
  const int64_t per = (p.T + BL - 1) / BL;
  return p.cu_seqlens ? per + p.n_seq : (int64_t)p.B * per;
}

// The blocks come first, one slot of layout(BL).block bytes per (block, head); the factored
// blocks (flayout().block bytes, one-chunk walks only) are packed at their own stride inside
// the same span, so the tables after it do not depend on the block format.
size_t block_table_offset(const ChunkPlan& p) {
  return (size_t)max_blocks(p) * p.H * layout(walk_block(p)).block;
}

// packed sequences: block offsets, then checkpoint offsets, then the order, after the blocks
size_t table_bytes(const ChunkPlan& p) { return ((sizeof(int32_t) * (p.n_seq + 1) + 255) / 256) * 256; }

}  // namespace

bool fast_path_applies(const ChunkPlan& p) {
  return p.act_bf16 && p.dk == DK && p.dv == DV && p.chunk == C;
}

namespace {
// Segmented walk: P - 1 entry states, and P - 2 summaries and transitions, after the tables.
int n_segments(const ChunkPlan& p) { return p.segments >= 3 ? p.segments : 1; }
size_t state_bytes(const ChunkPlan& p) { return (size_t)p.n_seq * p.H * DK * DV * sizeof(float); }
size_t segment_buffers_offset(const ChunkPlan& p) {
  return block_table_offset(p) + (p.cu_seqlens ? 3 * table_bytes(p) : 0);
}
}  // namespace

size_t fast_workspace_bytes(const ChunkPlan& p) {
  const int P = n_segments(p);
  return segment_buffers_offset(p) + (P > 1 ? (size_t)(3 * P - 5) * state_bytes(p) : 0);
}

namespace {

template <typename TOut, int BL>
hipError_t launch_rec(const ChunkPlan& p, hipStream_t stream, int strips, int halves, int64_t pairs,
                      RecJobs jobs, int n_jobs, const int32_t* blk_off,
                      const int32_t* ckpt_off, const int32_t* order, uint8_t* ws) {
  jobs.halves = halves;
  jobs.blocks_per_job = ((pairs + 7) / 8) * 8 * (NSTRIP / strips) * halves;
  const dim3 grid((unsigned)(jobs.blocks_per_job * n_jobs)), block(512);
  const int ck_blocks = p.ckpt ? p.ckpt_every / BL : 0;
  auto kern = p.ckpt ? (strips == 4   ? rec_kernel<TOut, 4, BL, true>
                        : strips == 2 ? rec_kernel<TOut, 2, BL, true>
                                      : rec_kernel<TOut, 1, BL, true>)
                     : (strips == 4   ? rec_kernel<TOut, 4, BL, false>
                        : strips == 2 ? rec_kernel<TOut, 2, BL, false>
                                      : rec_kernel<TOut, 1, BL, false>);
  hipLaunchKernelGGL(kern, grid, block, 0, stream, jobs, static_cast<TOut*>(p.o), p.cu_seqlens,
                     blk_off, p.T, p.H, p.n_seq, max_blocks(p), ws, p.ckpt, ck_blocks,
                     p.ckpt_slots, ckpt_off, order);
  return hipGetLastError();
}

template <typename TOut>
hipError_t launch_rec_fact(const ChunkPlan& p, hipStream_t stream, int strips, int halves,
                           int64_t pairs, RecJobs jobs, int n_jobs, const int32_t* blk_off,
                           const int32_t* ckpt_off, const int32_t* order, uint8_t* ws) {
  jobs.halves = halves;
  jobs.blocks_per_job = ((pairs + 7) / 8) * 8 * (NSTRIP / strips) * halves;
  const dim3 grid((unsigned)(jobs.blocks_per_job * n_jobs)), block(512);
  const int ck_blocks = p.ckpt ? p.ckpt_every / C : 0;
  auto kern = p.ckpt ? (strips == 4   ? rec_fact_kernel<TOut, 4, true>
                        : strips == 2 ? rec_fact_kernel<TOut, 2, true>
                                      : rec_fact_kernel<TOut, 1, true>)
                     : (strips == 4   ? rec_fact_kernel<TOut, 4, false>
                        : strips == 2 ? rec_fact_kernel<TOut, 2, false>
                                      : rec_fact_kernel<TOut, 1, false>);
  hipLaunchKernelGGL(kern, grid, block, 0, stream, jobs, static_cast<TOut*>(p.o), p.cu_seqlens,
                     blk_off, p.T, p.H, p.n_seq, max_blocks(p), ws, p.ckpt, ck_blocks,
                     p.ckpt_slots, ckpt_off, order);
  return hipGetLastError();
}

template <bool COMPOSE, bool FACT = false>
hipError_t launch_prep(const ChunkPlan& p, hipStream_t stream, const int32_t* blk_off, uint8_t* ws) {
  const int64_t blocks = max_blocks(p) * p.H;
  auto kern = p.pairwise_diag ? prep_kernel<true, COMPOSE, FACT> : prep_kernel<false, COMPOSE, FACT>;
  if (blocks > 0)
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(COMPOSE ? 512 : 256), 0, stream,
                       static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k),
                       static_cast<const uint16_t*>(p.v), static_cast<const uint16_t*>(p.g),
                       static_cast<const uint16_t*>(p.beta), p.cu_seqlens, blk_off, p.T, p.H,
                       p.n_seq, ws);
  return hipGetLastError();
}

template <int BL>
hipError_t launch_fast(const ChunkPlan& p, hipStream_t stream) {
  uint8_t* ws = static_cast<uint8_t*>(p.workspace);
  int32_t *blk_off = nullptr, *ckpt_off = nullptr, *order = nullptr;
  if (p.cu_seqlens) {
    blk_off = reinterpret_cast<int32_t*>(ws + block_table_offset(p));
    ckpt_off = reinterpret_cast<int32_t*>(ws + block_table_offset(p) + table_bytes(p));
    order = reinterpret_cast<int32_t*>(ws + block_table_offset(p) + 2 * table_bytes(p));
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, p.cu_seqlens, p.n_seq, p.T, BL,
                       p.ckpt ? p.ckpt_every : 0, blk_off, ckpt_off, order);
  }
  const int64_t pairs = (int64_t)p.n_seq * p.H;
  int dev = 0, n_cu = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  // Few (sequence, head) pairs: the chunk walk is latency bound, so one 16-column strip per
  // workgroup maximises parallelism. At least one strip per CU: two strips per workgroup halve
  // the state operand traffic per column (the walk is bound by each CU's vector memory unit);
  // measured faster from one strip per CU on (prefill-64k-bound -1.5 %); four from four strips
  // per CU on.
  const WalkShape shape = walk_shape(pairs, n_cu, p.S0 != nullptr && p.S0 == p.S_T);
  const int strips = shape.strips;
  // From one 16-column strip per CU on, the walk streams its operands at what HBM delivers
  // and its chain latency is hidden: then the factored block (98,816 of each block slot's
  // 114,688 bytes, and fewer products in prep) pays for the walk's second exchange per chunk
  // (prefill-64k-bound -2.7 %, varlen-16 -8.7 %). With fewer pairs the walk is latency bound
  // and one exchange per chunk wins.
  const bool fact = BL == C && strips >= 2;
  hipError_t e = fact ? launch_prep<false, true>(p, stream, blk_off, ws)
                      : launch_prep<BL == 2 * C>(p, stream, blk_off, ws);
  if (e != hipSuccess) return e;
  auto rec = [&](const RecJobs& jobs, int n_jobs, int halves) {
    if (fact)
      return p.out_bf16 ? launch_rec_fact<uint16_t>(p, stream, strips, halves, pairs, jobs, n_jobs, blk_off, ckpt_off, order, ws)
                        : launch_rec_fact<float>(p, stream, strips, halves, pairs, jobs, n_jobs, blk_off, ckpt_off, order, ws);
    return p.out_bf16 ? launch_rec<uint16_t, BL>(p, stream, strips, halves, pairs, jobs, n_jobs, blk_off, ckpt_off, order, ws)
                      : launch_rec<float, BL>(p, stream, strips, halves, pairs, jobs, n_jobs, blk_off, ckpt_off, order, ws);
  };
  RecJobs jobs = {};
  const int P = n_segments(p);
  if (P == 1) {  // one walk over every block
    jobs.job[0] = RecJob{0, INT64_MAX, p.S0, p.S_T, REC_OUTPUT};
    // The walk is bound by each CU's vector memory unit (the operand bytes per step). When
    // the walks would leave at least half of the CUs idle, two workgroups per walk run the
    // same state walk and split the output rows, so each loads the state operands and half of
    // the output operands (never in place: see walk_shape).
    return rec(jobs, 1, shape.halves);
  }
  // Segmented walk (sequence split of the transition form): the blocks of each sequence are
  // cut at b_1 < ... < b_{P-1}. Pass 1 walks segment 0 from S0 (its exit is segment 1's entry)
  // and, at the same time, every middle segment p from zeros (Z_p) and from the identity with
  // V = 0 (Phi_p). Then entry_{p+1} = Phi_p entry_p + Z_p, in order. Pass 2 walks segments
  // 1 .. P-1 from their entries, all at once.
  const int64_t span = ((p.T + BL - 1) / BL + P - 1) / P;  // blocks per segment (T bounds any sequence)
  float* buf = reinterpret_cast<float*>(ws + segment_buffers_offset(p));
  const size_t ns = state_bytes(p) / sizeof(float);
  auto entry = [&](int q) { return buf + (size_t)(q - 1) * ns; };                   // q = 1 .. P-1
  auto summ = [&](int q) { return buf + (size_t)(P - 1 + q - 1) * ns; };            // q = 1 .. P-2
  auto trans = [&](int q) { return buf + (size_t)(P - 1 + P - 2 + q - 1) * ns; };   // q = 1 .. P-2
  int n = 0;
  jobs.job[n++] = RecJob{0, span, p.S0, entry(1), REC_OUTPUT};
  for (int q = 1; q <= P - 2; ++q) {
    jobs.job[n++] = RecJob{q * span, (q + 1) * span, nullptr, summ(q), REC_SUMMARY};
    jobs.job[n++] = RecJob{q * span, (q + 1) * span, nullptr, trans(q), REC_TRANSITION};
  }
  if ((e = rec(jobs, n, 1)) != hipSuccess) return e;
  for (int q = 1; q <= P - 2; ++q) {
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(pairs * NSTRIP)), dim3(256), 0, stream,
                       trans(q), entry(q), summ(q), entry(q + 1), pairs);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  n = 0;
  for (int q = 1; q <= P - 1; ++q)
    jobs.job[n++] = RecJob{q * span, q == P - 1 ? INT64_MAX : (q + 1) * span, entry(q),
                           q == P - 1 ? p.S_T : nullptr, REC_OUTPUT};
  return rec(jobs, n, 1);
}

}  // namespace

hipError_t launch_chunk_fast(const ChunkPlan& p, hipStream_t stream) {
  return walk_block(p) == 2 * C ? launch_fast<2 * C>(p, stream) : launch_fast<C>(p, stream);
}

}  // namespace kda
