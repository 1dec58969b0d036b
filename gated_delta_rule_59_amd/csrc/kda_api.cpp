// libkda C ABI: argument validation, path selection, workspace sizing and launches.
// Every check happens on the host before anything is enqueued; see include/kda.h.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <string>

#include "kda_internal.h"

namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

kda_status ok() {
  g_last_error.clear();
  return KDA_OK;
}

// A launch's grid holds at most 2^32 - 1 work-items. The decode kernels run one
// 256-work-item workgroup per (sequence, head).
constexpr int64_t kMaxGridItems = 0xffffffffLL;
constexpr int64_t kMaxDecodePairs = kMaxGridItems / 256;

bool head_dim_ok(int d) { return d == 32 || d == 64 || d == 128; }
bool dtype_ok(kda_dtype t) { return t == KDA_F32 || t == KDA_BF16; }
size_t dsize(kda_dtype t) { return t == KDA_F32 ? 4 : 2; }

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char* name, const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{name, a, a + bytes};
}

bool overlap(const Range& a, const Range& b) {
  return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo;
}

bool env_check() {
  const char* s = std::getenv("KDA_CHECK");
  return s && s[0] == '1';
}

// Counts g outside [-5, 0] and beta outside [0, 1] on the device into counts[0 .. n_counts)
// (caller-owned device memory; at most kda::check_blocks() of them are used), copies them to
// the host and synchronises the stream.
kda_status run_gate_check(const void* g, int64_t n_g, const void* beta, int64_t n_beta,
                          kda_dtype dt, int64_t* counts, int64_t n_counts, hipStream_t stream,
                          int64_t* n_bad) {
  int64_t host[1024];
  static_assert(sizeof(host) / sizeof(host[0]) >= 1024, "host copy of the counters");
  const int nb = (int)std::min<int64_t>(n_counts, kda::check_blocks());
  hipError_t e = kda::launch_check_gates(g, n_g, beta, n_beta, dt == KDA_BF16, counts, nb, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(host, counts, sizeof(int64_t) * nb, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "gate check: %s", hipGetErrorString(e));
  int64_t total = 0;
  for (int i = 0; i < nb; ++i) total += host[i];
  *n_bad = total;
  return ok();
}

// KDA_CHECK=1: the gate check before a call, its counters held in the call's output buffer o
// (which the call overwrites afterwards, and which overlaps no input), so that nothing is
// allocated. o_bytes >= 64 (one token of one head), so at least seven 8-byte aligned
// counters fit.
kda_status env_gate_check(const void* g, int64_t n_g, const void* beta, int64_t n_beta,
                          kda_dtype dt, void* o, size_t o_bytes, hipStream_t stream) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(o), end = lo + o_bytes;
  const uintptr_t c0 = (lo + 7) & ~uintptr_t(7);
  int64_t bad = 0;
  kda_status s = run_gate_check(g, n_g, beta, n_beta, dt, reinterpret_cast<int64_t*>(c0),
                                (int64_t)((end - c0) / sizeof(int64_t)), stream, &bad);
  if (s != KDA_OK) return s;
  if (bad) return fail(KDA_ERR_DECAY_RANGE, "%lld gate values outside their range", (long long)bad);
  return KDA_OK;
}

// Tokens per step of the matrix-core walk. Two chunks composed into one 128-token step halve
// the serial steps and the workspace bytes, but the composition costs the parallel part about
// 30 % more; measured on MI355X it pays where the walk dominates, i.e. few (sequence, head)
// pairs (one 65,536-token sequence: 0.708 -> 0.446 ms with 2 heads, 1.12 -> 1.00 ms with 8),
// and is even with 16 or 32 heads. One chunk per step when asked, and whenever checkpoints fall
// between 128-token steps (decided from ckpt_every alone, so that the workspace size does not
// depend on ckpt_slots).
constexpr int kComposeMaxPairs = 8;
int walk_block(const kda_chunk_args* a, int n_seq) {
  if ((a->flags & KDA_FLAG_WALK64) || (a->ckpt_every > 0 && a->ckpt_every % 128 != 0)) return 64;
  if (a->flags & KDA_FLAG_WALK128) return 128;
  return (int64_t)n_seq * a->H <= kComposeMaxPairs ? 128 : 64;
}

// Shape/dtype validation shared by kda_chunk_fwd and kda_chunk_fwd_workspace_bytes.
kda_status validate_chunk_shapes(const kda_chunk_args* a, kda::ChunkPlan* p) {
  if (!a) return fail(KDA_ERR_NULL_PTR, "args is NULL");
  if (a->B < 1 || a->T < 0 || a->H < 1)
    return fail(KDA_ERR_BAD_SHAPE, "need B >= 1, T >= 0, H >= 1 (got B=%d T=%d H=%d)", a->B, a->T,
                a->H);
  if (!head_dim_ok(a->dk) || !head_dim_ok(a->dv))
    return fail(KDA_ERR_BAD_SHAPE, "dk and dv must be 32, 64 or 128 (got %d, %d)", a->dk, a->dv);
  if (a->chunk != 16 && a->chunk != 32 && a->chunk != 64)
    return fail(KDA_ERR_BAD_SHAPE, "chunk must be 16, 32 or 64 (got %d)", a->chunk);
  if (a->cu_seqlens) {
    if (a->B != 1) return fail(KDA_ERR_BAD_SHAPE, "cu_seqlens requires B == 1 (got %d)", a->B);
    if (a->N < 1) return fail(KDA_ERR_BAD_SHAPE, "cu_seqlens requires N >= 1 (got %d)", a->N);
  }
  if (!dtype_ok(a->act_dtype) || !dtype_ok(a->gate_dtype) || !dtype_ok(a->out_dtype))
    return fail(KDA_ERR_BAD_DTYPE, "unknown dtype");
  if (a->act_dtype != a->gate_dtype)
    return fail(KDA_ERR_BAD_DTYPE, "act_dtype and gate_dtype must match (both F32 or both BF16)");
  if (a->flags & ~(KDA_FLAG_GENERIC | KDA_FLAG_PAIRWISE_DIAG | KDA_FLAG_WALK64 | KDA_FLAG_WALK128))
    return fail(KDA_ERR_UNSUPPORTED, "unknown flags 0x%x", a->flags);
  if ((a->flags & KDA_FLAG_WALK64) && (a->flags & KDA_FLAG_WALK128))
    return fail(KDA_ERR_UNSUPPORTED, "KDA_FLAG_WALK64 and KDA_FLAG_WALK128 exclude each other");
  if ((a->flags & KDA_FLAG_WALK128) && a->ckpt_every > 0 && a->ckpt_every % 128 != 0)
    return fail(KDA_ERR_UNSUPPORTED,
                "KDA_FLAG_WALK128: checkpoints every %d tokens fall between 128-token steps",
                a->ckpt_every);
  const int64_t tokens = (int64_t)a->B * a->T;
  const int n_seq = a->cu_seqlens ? a->N : a->B;
  if (tokens * a->H * (int64_t)(a->dk > a->dv ? a->dk : a->dv) > (int64_t(1) << 40))
    return fail(KDA_ERR_BAD_SHAPE, "problem too large");
  if ((int64_t)n_seq * a->H * (a->dv / 16) > 0x7fffffffLL)
    return fail(KDA_ERR_BAD_SHAPE, "too many (sequence, head) pairs");
  // the largest grid either prefill path launches (work-items): the per-(chunk, head)
  // kernel, and the walk's (sequence, head, column strip) workgroups of up to 512 work-items,
  // two per strip, for each of up to 15 segment walks
  const int64_t chunks = (a->cu_seqlens ? ((int64_t)a->T + 63) / 64 + n_seq
                                        : (int64_t)a->B * (((int64_t)a->T + 63) / 64));
  const int64_t walk_items = ((int64_t)n_seq * a->H + 7) / 8 * 8 * (a->dv / 16) * 2 * 512 *
                             (a->segments >= 3 ? 2 * a->segments - 3 : 1);
  if (chunks * a->H * 256 > kMaxGridItems || walk_items > kMaxGridItems)
    return fail(KDA_ERR_BAD_SHAPE, "the problem needs more work-items than one launch holds");
  if (a->ckpt_every < 0 || (a->ckpt_every > 0 && a->ckpt_every % a->chunk != 0))
    return fail(KDA_ERR_BAD_SHAPE, "ckpt_every must be 0 or a positive multiple of chunk (got %d)",
                a->ckpt_every);
  if (a->ckpt_every > 0 && a->ckpt_slots < 0)
    return fail(KDA_ERR_BAD_SHAPE, "ckpt_slots must be >= 0 (got %d)", a->ckpt_slots);
  if (a->segments < 0 || a->segments > 8)
    return fail(KDA_ERR_BAD_SHAPE, "segments must be in 0 .. 8 (got %d)", a->segments);
  const bool ck = a->ckpt_every > 0 && a->ckpt_slots > 0;
  *p = kda::ChunkPlan{a->B, a->T, a->H, a->dk, a->dv, a->chunk, a->cu_seqlens, n_seq,
                      a->act_dtype == KDA_BF16, a->out_dtype == KDA_BF16,
                      a->q, a->k, a->v, a->g, a->beta, a->S0, a->o, a->S_T,
                      a->workspace, a->workspace_bytes,
                      ck ? a->ckpt : nullptr, ck ? a->ckpt_every : 0, ck ? a->ckpt_slots : 0,
                      (a->flags & KDA_FLAG_PAIRWISE_DIAG) != 0, a->segments,
                      walk_block(a, n_seq)};
  return KDA_OK;
}

bool use_fast(const kda_chunk_args* a, const kda::ChunkPlan& p) {
  return !(a->flags & KDA_FLAG_GENERIC) && kda::fast_path_applies(p);
}

// kda_chunk_fwd and kda_chunk_fwd_noalloc. With noalloc the workspace fields of *a are
// ignored and the library's fixed device scratch takes the workspace's place.
kda_status chunk_fwd(const kda_chunk_args* a, void* hip_stream, bool noalloc) {
  kda::ChunkPlan p;
  kda_status s = validate_chunk_shapes(a, &p);
  if (s != KDA_OK) return s;
  const size_t es = dsize(a->act_dtype), os = dsize(a->out_dtype);
  const size_t tok = (size_t)a->B * a->T * a->H;
  // zero tokens: the per-token arrays are empty and may be NULL (as an empty tensor's is)
  if (tok > 0 && (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->o))
    return fail(KDA_ERR_NULL_PTR, "q, k, v, g, beta and o must be non-NULL");
  const size_t st = (size_t)p.n_seq * a->H * a->dk * a->dv * 4;
  const Range in[] = {range("q", a->q, tok * a->dk * es), range("k", a->k, tok * a->dk * es),
                      range("v", a->v, tok * a->dv * es), range("g", a->g, tok * a->dk * es),
                      range("beta", a->beta, tok * es),
                      range("S0", a->S0, a->S0 ? st : 0),
                      range("cu_seqlens", a->cu_seqlens,
                            a->cu_seqlens ? sizeof(int32_t) * (a->N + 1) : 0)};
  const Range o = range("o", a->o, tok * a->dv * os);
  const Range sT = range("S_T", a->S_T, a->S_T ? st : 0);
  for (const Range& r : in)
    if (overlap(o, r)) return fail(KDA_ERR_ALIAS, "o overlaps %s", r.name);
  for (const Range& r : in) {
    if (!overlap(sT, r)) continue;
    if (std::strcmp(r.name, "S0") == 0 && a->S_T == a->S0) continue;  // in-place continue
    return fail(KDA_ERR_ALIAS, "S_T overlaps %s", r.name);
  }
  if (overlap(sT, o)) return fail(KDA_ERR_ALIAS, "S_T overlaps o");
  if (p.ckpt_every > 0 && !a->ckpt) return fail(KDA_ERR_NULL_PTR, "ckpt is NULL with ckpt_every > 0");
  const Range ck = range("ckpt", p.ckpt, p.ckpt ? (size_t)p.ckpt_slots * a->H * a->dk * a->dv * 4 : 0);
  for (const Range& r : in)
    if (overlap(ck, r)) return fail(KDA_ERR_ALIAS, "ckpt overlaps %s", r.name);
  if (overlap(ck, o) || overlap(ck, sT)) return fail(KDA_ERR_ALIAS, "ckpt overlaps an output");

  const bool fast = use_fast(a, p);
  if (fast && noalloc) {
    const size_t need = kda::fast_workspace_bytes(p);
    if (need > kda::noalloc_scratch_bytes())
      return fail(KDA_ERR_WORKSPACE,
                  "kda_chunk_fwd_noalloc: these sizes need %zu bytes of scratch, more than the "
                  "%zu bytes of the library's fixed scratch (use kda_chunk_fwd with a workspace)",
                  need, kda::noalloc_scratch_bytes());
    void* ws = nullptr;
    const hipError_t e = kda::noalloc_scratch(&ws);
    if (e != hipSuccess)
      return fail(KDA_ERR_HIP, "kda_chunk_fwd_noalloc: scratch address: %s", hipGetErrorString(e));
    p.workspace = ws;
    p.workspace_bytes = kda::noalloc_scratch_bytes();
  } else if (fast) {
    const size_t need = kda::fast_workspace_bytes(p);
    if (need && (!a->workspace || a->workspace_bytes < need))
      return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  a->workspace ? a->workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(a->workspace) % 256)
      return fail(KDA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    const Range ws = range("workspace", a->workspace, need);
    for (const Range& r : in)
      if (overlap(ws, r)) return fail(KDA_ERR_ALIAS, "workspace overlaps %s", r.name);
    if (overlap(ws, o) || overlap(ws, sT) || overlap(ws, ck))
      return fail(KDA_ERR_ALIAS, "workspace overlaps an output");
  }
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (env_check() && tok > 0) {
    s = env_gate_check(a->g, (int64_t)(tok * a->dk), a->beta, (int64_t)tok, a->gate_dtype, a->o,
                       tok * a->dv * os, stream);
    if (s != KDA_OK) return s;
  }
  const hipError_t e = fast ? kda::launch_chunk_fast(p, stream) : kda::launch_chunk_generic(p, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "kda_chunk_fwd launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd(const kda_chunk_args* a, void* hip_stream) {
  return chunk_fwd(a, hip_stream, false);
}

kda_status kda_chunk_fwd_noalloc(const kda_chunk_args* a, void* hip_stream) {
  return chunk_fwd(a, hip_stream, true);
}

size_t kda_chunk_fwd_workspace_bytes(const kda_chunk_args* a) {
  kda::ChunkPlan p;
  if (validate_chunk_shapes(a, &p) != KDA_OK) return SIZE_MAX;
  ok();
  return use_fast(a, p) ? kda::fast_workspace_bytes(p) : 0;
}

kda_status kda_decode_step(const kda_decode_args* a, void* hip_stream) {
  if (!a) return fail(KDA_ERR_NULL_PTR, "args is NULL");
  if (a->N < 1 || a->H < 1)
    return fail(KDA_ERR_BAD_SHAPE, "need N >= 1 and H >= 1 (got N=%d H=%d)", a->N, a->H);
  if (!head_dim_ok(a->dk) || !head_dim_ok(a->dv))
    return fail(KDA_ERR_BAD_SHAPE, "dk and dv must be 32, 64 or 128 (got %d, %d)", a->dk, a->dv);
  if ((int64_t)a->N * a->H > kMaxDecodePairs)
    return fail(KDA_ERR_BAD_SHAPE, "N * H = %lld exceeds one launch (%lld)",
                (long long)a->N * a->H, (long long)kMaxDecodePairs);
  if (!dtype_ok(a->act_dtype) || !dtype_ok(a->gate_dtype) || !dtype_ok(a->out_dtype))
    return fail(KDA_ERR_BAD_DTYPE, "unknown dtype");
  if (a->act_dtype != a->gate_dtype)
    return fail(KDA_ERR_BAD_DTYPE, "act_dtype and gate_dtype must match (both F32 or both BF16)");
  if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->S || !a->o)
    return fail(KDA_ERR_NULL_PTR, "q, k, v, g, beta, S and o must be non-NULL");
  const size_t es = dsize(a->act_dtype), os = dsize(a->out_dtype);
  const size_t nh = (size_t)a->N * a->H;
  const Range in[] = {range("q", a->q, nh * a->dk * es), range("k", a->k, nh * a->dk * es),
                      range("v", a->v, nh * a->dv * es), range("g", a->g, nh * a->dk * es),
                      range("beta", a->beta, nh * es)};
  const Range S = range("S", a->S, nh * a->dk * a->dv * 4);
  const Range o = range("o", a->o, nh * a->dv * os);
  for (const Range& r : in) {
    if (overlap(o, r)) return fail(KDA_ERR_ALIAS, "o overlaps %s", r.name);
    if (overlap(S, r)) return fail(KDA_ERR_ALIAS, "S overlaps %s", r.name);
  }
  if (overlap(S, o)) return fail(KDA_ERR_ALIAS, "S overlaps o");
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (env_check()) {
    kda_status s = env_gate_check(a->g, (int64_t)(nh * a->dk), a->beta, (int64_t)nh,
                                  a->gate_dtype, a->o, nh * a->dv * os, stream);
    if (s != KDA_OK) return s;
  }
  const kda::DecodePlan p{a->N, a->H, a->dk, a->dv, a->act_dtype == KDA_BF16,
                          a->out_dtype == KDA_BF16, a->q, a->k, a->v, a->g, a->beta, a->S, a->o};
  const hipError_t e = kda::launch_decode(p, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "kda_decode_step launch: %s", hipGetErrorString(e));
  return ok();
}

kda_status kda_decode_multi(const kda_decode_multi_args* a, void* hip_stream) {
  if (!a) return fail(KDA_ERR_NULL_PTR, "args is NULL");
  if (a->N < 1 || a->H < 1 || a->m < 1)
    return fail(KDA_ERR_BAD_SHAPE, "need N, H, m >= 1 (got N=%d H=%d m=%d)", a->N, a->H, a->m);
  if (!head_dim_ok(a->dk) || !head_dim_ok(a->dv))
    return fail(KDA_ERR_BAD_SHAPE, "dk and dv must be 32, 64 or 128 (got %d, %d)", a->dk, a->dv);
  if ((int64_t)a->N * a->H > kMaxDecodePairs || (int64_t)a->N * a->m * a->H > (int64_t(1) << 40))
    return fail(KDA_ERR_BAD_SHAPE, "N * H or N * m * H too large for one launch");
  if (!dtype_ok(a->act_dtype) || !dtype_ok(a->gate_dtype) || !dtype_ok(a->out_dtype))
    return fail(KDA_ERR_BAD_DTYPE, "unknown dtype");
  if (a->act_dtype != a->gate_dtype)
    return fail(KDA_ERR_BAD_DTYPE, "act_dtype and gate_dtype must match (both F32 or both BF16)");
  if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->S)
    return fail(KDA_ERR_NULL_PTR, "q, k, v, g, beta and S must be non-NULL");
  const size_t es = dsize(a->act_dtype), os = dsize(a->out_dtype);
  const size_t nh = (size_t)a->N * a->H, nmh = nh * a->m;
  const Range in[] = {range("q", a->q, nmh * a->dk * es), range("k", a->k, nmh * a->dk * es),
                      range("v", a->v, nmh * a->dv * es), range("g", a->g, nmh * a->dk * es),
                      range("beta", a->beta, nmh * es),
                      range("accept", a->accept, a->accept ? sizeof(int32_t) * a->N : 0)};
  const Range S = range("S", a->S, nh * a->dk * a->dv * 4);
  const Range o = range("o", a->o, a->o ? nmh * a->dv * os : 0);
  for (const Range& r : in) {
    if (overlap(o, r)) return fail(KDA_ERR_ALIAS, "o overlaps %s", r.name);
    if (overlap(S, r)) return fail(KDA_ERR_ALIAS, "S overlaps %s", r.name);
  }
  if (overlap(S, o)) return fail(KDA_ERR_ALIAS, "S overlaps o");
  if (!a->o && !a->accept) return ok();
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (env_check()) {
    if (!a->o)
      return fail(KDA_ERR_UNSUPPORTED, "KDA_CHECK=1 needs o (the check keeps its counters there)");
    kda_status s = env_gate_check(a->g, (int64_t)(nmh * a->dk), a->beta, (int64_t)nmh,
                                  a->gate_dtype, a->o, nmh * a->dv * os, stream);
    if (s != KDA_OK) return s;
  }
  const kda::DecodeMultiPlan p{a->N, a->H, a->dk, a->dv, a->m, a->act_dtype == KDA_BF16,
                               a->out_dtype == KDA_BF16, a->q, a->k, a->v, a->g, a->beta,
                               a->S, a->o, a->accept};
  const hipError_t e = kda::launch_decode_multi(p, stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "kda_decode_multi launch: %s", hipGetErrorString(e));
  return ok();
}

kda_status kda_check_gates(const void* g, int64_t n_g, const void* beta, int64_t n_beta,
                           kda_dtype gate_dtype, int64_t* counts, int n_counts,
                           void* hip_stream, int64_t* n_bad) {
  if (!n_bad) return fail(KDA_ERR_NULL_PTR, "n_bad is NULL");
  if (n_g < 0 || n_beta < 0) return fail(KDA_ERR_BAD_SHAPE, "negative element count");
  if ((n_g && !g) || (n_beta && !beta)) return fail(KDA_ERR_NULL_PTR, "g or beta is NULL");
  if (!counts) return fail(KDA_ERR_NULL_PTR, "counts is NULL");
  if (n_counts < 1) return fail(KDA_ERR_BAD_SHAPE, "n_counts must be >= 1 (got %d)", n_counts);
  if (!dtype_ok(gate_dtype)) return fail(KDA_ERR_BAD_DTYPE, "unknown dtype");
  const size_t es = dsize(gate_dtype);
  const size_t used = sizeof(int64_t) * (size_t)std::min(n_counts, kda::check_blocks());
  const Range c = range("counts", counts, used);
  if (overlap(c, range("g", g, (size_t)n_g * es)) || overlap(c, range("beta", beta, (size_t)n_beta * es)))
    return fail(KDA_ERR_ALIAS, "counts overlaps g or beta");
  return run_gate_check(g, n_g, beta, n_beta, gate_dtype, counts, n_counts,
                        static_cast<hipStream_t>(hip_stream), n_bad);
}

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL_PTR: return "KDA_ERR_NULL_PTR";
    case KDA_ERR_BAD_SHAPE: return "KDA_ERR_BAD_SHAPE";
    case KDA_ERR_BAD_DTYPE: return "KDA_ERR_BAD_DTYPE";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_DECAY_RANGE: return "KDA_ERR_DECAY_RANGE";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS";
  }
  return "KDA_ERR_UNKNOWN";
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

int kda_abi_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"
