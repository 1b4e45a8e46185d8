// C-ABI front end: host-side argument checks, then one launch on the caller's
// stream. Every check runs before any HIP call, so the error paths need no GPU.
#include <cstdint>
#include <cstdio>
#include <cstddef>
#include <numeric>

#include "internal.h"
#include "lightning.h"

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
    bool empty() const { return hi <= lo; }
};

Range range_of(const void *p, long long bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, bytes > 0 ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool overlaps(Range a, Range b) {
    if (a.empty() || b.empty()) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool dtype_ok(int d) { return d == LT_F32 || d == LT_BF16; }
long long dtype_size(int d) { return d == LT_F32 ? 4 : 2; }

// a * b * c * d as 64-bit with overflow detection (all operands >= 0).
bool mul4(long long a, long long b, long long c, long long d, long long *out) {
    long long t;
    if (__builtin_mul_overflow(a, b, &t)) return false;
    if (__builtin_mul_overflow(t, c, &t)) return false;
    if (__builtin_mul_overflow(t, d, &t)) return false;
    *out = t;
    return true;
}

// A failed launch is reported as LT_ERR_HIP; the HIP error itself goes to
// stderr, the only place the status code cannot carry it.
lt_status map_hip(hipError_t e) {
    if (e == hipSuccess) return LT_OK;
    std::fprintf(stderr, "liblightning: kernel launch failed: %s (%d)\n", hipGetErrorName(e), (int)e);
    return LT_ERR_HIP;
}

// Workgroups a prefill launch should reach to occupy MI355X (256 CUs; the
// whole-head kernel runs one 8-wave workgroup per CU).
constexpr long long kTargetWorkgroups = 256;
// Shortest segment worth a workgroup of its own.
constexpr long long kMinSegment = 2048;
// Pre-pass pieces to plan for (the pieces cover the first G-1 segments of
// every head; heads on warm-up ranges skip them, and when many heads do take
// the pre-pass the kernels merge consecutive pieces into groups so that
// about 512 workgroups work). Fine pieces suit the case of few pre-pass heads
// (measured on the M1 layer when 7 of its 64 heads took it: 512 -> 661 us,
// 1024 -> 643 us, 2048 -> 608 us per call).
constexpr long long kPrepassWide = 2048;
// Shortest pre-pass piece.
constexpr long long kMinPiece = 512;

// need_ws: fail with LT_ERR_SCRATCH instead of running without segments when a
// segmented plan does not fit the workspace (the no-allocation entry point).
lt_status launch(const lt::PrefillArgs &a, int in_dtype, int out_dtype, bool varlen,
                 void *workspace, size_t workspace_bytes, void *stream, bool need_ws = false) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (in_dtype != LT_BF16)
        return map_hip(lt::launch_prefill_slices(a, (lt_dtype)in_dtype, (lt_dtype)out_dtype, st));
    const bool whole_rows = a.ng.gate || a.state_in_t;  // epilogue or transposed S_0
    // packed batches plan on their longest sequence (a.seqlen = max_seqlen)
    lt::PrefillPlan p = lt::plan_prefill(a.units, a.seqlen, a.heads, (lt_dtype)in_dtype, varlen,
                                         kPrepassWide, workspace ? workspace_bytes : 0);
    if (p.workspace_short && need_ws) return LT_ERR_SCRATCH;
    // Without a workspace for any segmented plan, value columns are split
    // instead; the norm-gate epilogue needs whole output rows, so it keeps one
    // workgroup per (sequence, head) rather than value slices.
    if (whole_rows && p.value_slices != 1) p = lt::PrefillPlan{};
    // one segment covers any sequence of the call (for packed batches whatever
    // the lengths on the device are)
    if (p.segments == 1) p.seg_len = varlen ? a.total_tokens : a.seqlen;
    return map_hip(lt::launch_prefill_heads(a, p, workspace, (lt_dtype)out_dtype, st));
}

// Shared checks of the two prefill entry points. `tokens` = rows of q/k/v/o.
lt_status check_prefill(const void *q, const void *k, const void *v, int in_dtype,
                        const float *slopes, void *o, int out_dtype,
                        const float *state_in, float *state_out,
                        long long units, long long tokens, int heads, int head_dim,
                        int block) {
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return LT_ERR_DTYPE;
    if (head_dim != lt::kHeadDim || heads < 0 || heads > LT_MAX_HEADS || units < 0 || tokens < 0)
        return LT_ERR_SHAPE;
    if (block < 1 || block > LT_MAX_BLOCK) return LT_ERR_BLOCK;
    if (units == 0 || heads == 0) return LT_OK;
    if (!slopes) return LT_ERR_NULL;
    if (tokens > 0 && (!q || !k || !v || !o)) return LT_ERR_NULL;

    long long in_bytes, out_bytes, st_bytes, grid;
    if (!mul4(tokens, heads, head_dim, dtype_size(in_dtype), &in_bytes) ||
        !mul4(tokens, heads, head_dim, dtype_size(out_dtype), &out_bytes) ||
        !mul4(units, heads, (long long)head_dim * head_dim, 4, &st_bytes) ||
        !mul4(units, heads, lt::kValueSlices, 1, &grid) || grid > 0x7fffffffLL)
        return LT_ERR_SHAPE;

    const Range rq = range_of(q, in_bytes), rk = range_of(k, in_bytes),
                rv = range_of(v, in_bytes), ro = range_of(o, out_bytes),
                rs = range_of(slopes, (long long)heads * 4),
                rsi = range_of(state_in, state_in ? st_bytes : 0),
                rso = range_of(state_out, state_out ? st_bytes : 0);
    if (overlaps(ro, rq) || overlaps(ro, rk) || overlaps(ro, rv) || overlaps(ro, rs) ||
        overlaps(ro, rsi) || overlaps(ro, rso))
        return LT_ERR_ALIAS;
    if (overlaps(rso, rq) || overlaps(rso, rk) || overlaps(rso, rv) || overlaps(rso, rs))
        return LT_ERR_ALIAS;
    if (state_in && state_out && state_in != state_out && overlaps(rsi, rso))
        return LT_ERR_ALIAS;
    return LT_OK;
}

// Stride of the decode workgroup order: the integer nearest 0.618 * batch
// that is coprime with batch (so b -> b * stride mod batch is a bijection),
// the golden-ratio step that keeps consecutive workgroups' states far apart.
// Measured on the 256 x 64 batch: most strides give 0.357-0.361 ms per step,
// sequence order 0.380 ms, and strides = +-1 mod 32 (31, 33) only 0.370 ms.
int decode_seq_stride(int batch) {
    if (batch < 8) return 1;
    int p = (int)(0.6180339887 * batch + 0.5);
    while (std::gcd(p, batch) != 1) ++p;
    return p % batch;
}

// Checks of the norm-gate variants: eps, the gate and weight pointers (needed
// when there are tokens), and overlap of the outputs with them.
lt_status check_norm_gate(const void *gate, long long gate_bytes, const float *norm_weight,
                          float eps, int heads, int head_dim, const void *y, long long y_bytes,
                          const float *state_out, long long st_bytes) {
    if (!(eps >= 0.f) || eps == __builtin_inff()) return LT_ERR_VALUE;  // NaN fails eps >= 0
    if (gate_bytes > 0 && (!gate || !norm_weight)) return LT_ERR_NULL;
    const Range rg = range_of(gate, gate_bytes),
                rw = range_of(norm_weight, norm_weight ? (long long)heads * head_dim * 4 : 0),
                ry = range_of(y, y_bytes), rs = range_of(state_out, state_out ? st_bytes : 0);
    if (overlaps(ry, rg) || overlaps(ry, rw) || overlaps(rs, rg) || overlaps(rs, rw))
        return LT_ERR_ALIAS;
    return LT_OK;
}

}  // namespace

namespace lt {

PrefillPlan plan_prefill(long long units, long long seqlen, int heads, lt_dtype in_dtype,
                         bool varlen, long long prepass_wgs, size_t max_workspace) {
    // bf16 plans, by the number of (sequence, head) pairs uh:
    //   uh >= 256: one whole-head workgroup per pair;
    //   long sequences: whole heads cut into segments, with the pre-pass (its
    //     extra k, v reads cost less than re-reading q, k per
    //     value slice, which measured 4.05 TB/s memory-only against 5.2 TB/s);
    //     packed batches cut on their longest sequence (seqlen = max_seqlen),
    //     each sequence using the segments its own length needs;
    //   otherwise (short sequences): four value-slice workgroups per pair.
    (void)varlen;
    PrefillPlan p;
    p.seg_len = seqlen;
    if (in_dtype != LT_BF16 || units <= 0 || heads <= 0) return p;
    const long long uh = units * heads;
    if (uh >= kTargetWorkgroups) return p;
    p.value_slices = kValueSlices;
    long long g = (kTargetWorkgroups + uh - 1) / uh;
    if (g > seqlen / kMinSegment) g = seqlen / kMinSegment;
    if (g < 2) return p;
    long long seg = (seqlen + g - 1) / g;
    seg = (seg + 127) / 128 * 128;  // segmented kernels step two sub-blocks at a time
    g = (seqlen + seg - 1) / seg;
    if (g < 2) return p;
    // Pre-pass pieces over the first (g-1) segments. piece <= seg, so a piece
    // holds at most one segment boundary strictly inside it.
    const long long covered = (g - 1) * seg;
    const long long want = (prepass_wgs + uh - 1) / uh;
    long long piece = (covered + want - 1) / want;
    piece = (piece + 127) / 128 * 128;
    if (piece < kMinPiece) piece = kMinPiece;
    if (piece > seg) piece = seg;
    constexpr size_t kStateBytes = (size_t)kHeadDim * kHeadDim * sizeof(float);
    auto bytes = [&](long long pieces) {
        return (size_t)uh * (size_t)prefill_states((int)g, (int)pieces) * kStateBytes;
    };
    long long pieces = (covered + piece - 1) / piece;
    if (bytes(pieces) > max_workspace) {
        // longer pieces: as many states as fit (at least one piece per segment
        // boundary, i.e. pieces of a whole segment)
        const long long fit = (long long)(max_workspace / kStateBytes / (size_t)uh) - g;
        if (fit < g - 1) {
            p.workspace_short = true;
            return p;
        }
        piece = (covered + fit - 1) / fit;
        piece = (piece + 127) / 128 * 128;
        if (piece > seg) piece = seg;
        pieces = (covered + piece - 1) / piece;
    }
    p.value_slices = 1;
    p.segments = (int)g;
    p.seg_len = seg;
    p.piece_len = piece;
    p.pieces = (int)pieces;
    p.workspace = bytes(pieces);
    return p;
}

}  // namespace lt

extern "C" {

LT_API size_t lt_prefill_workspace_bytes(int batch, long long seqlen, int heads, int head_dim,
                                         lt_dtype in_dtype) {
    if (batch <= 0 || seqlen <= 0 || heads <= 0 || heads > LT_MAX_HEADS ||
        head_dim != lt::kHeadDim || !dtype_ok(in_dtype))
        return 0;
    return lt::plan_prefill(batch, seqlen, heads, in_dtype, false, kPrepassWide, SIZE_MAX).workspace;
}

LT_API size_t lt_prefill_varlen_workspace_bytes(int num_seqs, long long max_seqlen, int heads,
                                                int head_dim, lt_dtype in_dtype) {
    if (num_seqs <= 0 || max_seqlen <= 0 || heads <= 0 || heads > LT_MAX_HEADS ||
        head_dim != lt::kHeadDim || !dtype_ok(in_dtype))
        return 0;
    return lt::plan_prefill(num_seqs, max_seqlen, heads, in_dtype, true, kPrepassWide, SIZE_MAX).workspace;
}

LT_API const char *lt_status_string(int status) {
    switch (status) {
        case LT_OK: return "LT_OK";
        case LT_ERR_NULL: return "LT_ERR_NULL: a required pointer is NULL";
        case LT_ERR_SHAPE: return "LT_ERR_SHAPE: unsupported or inconsistent sizes";
        case LT_ERR_BLOCK: return "LT_ERR_BLOCK: block size out of range";
        case LT_ERR_DTYPE: return "LT_ERR_DTYPE: unsupported dtype";
        case LT_ERR_ALIAS: return "LT_ERR_ALIAS: an output overlaps another buffer";
        case LT_ERR_HIP: return "LT_ERR_HIP: HIP runtime error at launch";
        case LT_ERR_VALUE: return "LT_ERR_VALUE: a scalar argument is out of range";
        case LT_ERR_SCRATCH:
            return "LT_ERR_SCRATCH: the call needs more scratch than the no-allocation entry point holds";
        default: return "unknown lt_status";
    }
}

LT_API int lt_version(void) { return 20100; }

LT_API lt_status lt_init(void) {
    hipError_t (*const loads[])() = {lt::load_prefill_heads_code, lt::load_prefill_slices_code,
                                     lt::load_decode_code, lt::load_backward_code, lt::load_softmax_code};
    for (auto load : loads)
        if (load() != hipSuccess) return LT_ERR_HIP;
    void *scratch = nullptr;
    size_t bytes = 0;
    return lt::noalloc_scratch(nullptr, &scratch, &bytes) == hipSuccess ? LT_OK : LT_ERR_HIP;
}

// The build passes the hash of the sources it compiled; a build by other means
// reports "unknown". The tag keeps a fixed prefix so the identity can also be
// read from the library file without loading it.
#ifndef LT_BUILD_ID
#define LT_BUILD_ID "unknown"
#endif
static const char kBuildTag[] = "LT_BUILD_ID=" LT_BUILD_ID;
LT_API const char *lt_build_id(void) { return kBuildTag + sizeof("LT_BUILD_ID=") - 1; }

}  // extern "C"

namespace {

lt_status prefill_impl(const void *q, const void *k, const void *v, lt_dtype in_dtype,
                       const float *slopes, void *o, lt_dtype out_dtype, const float *state_in,
                       float *state_out, int batch, long long seqlen, int heads, int head_dim,
                       int block, void *workspace, size_t workspace_bytes, void *stream,
                       const lt::NormGate *ng, bool use_scratch = false) {
    if (batch < 0 || seqlen < 0) return LT_ERR_SHAPE;
    long long tokens;
    if (__builtin_mul_overflow((long long)batch, seqlen, &tokens)) return LT_ERR_SHAPE;
    lt_status st = check_prefill(q, k, v, in_dtype, slopes, o, out_dtype, state_in, state_out,
                                 batch, tokens, heads, head_dim, block);
    if (st != LT_OK) return st;
    const long long in_b = tokens * heads * head_dim * dtype_size(in_dtype);
    const long long st_b = (long long)batch * heads * head_dim * head_dim * 4;
    if (ng) {
        if (in_dtype != LT_BF16) return LT_ERR_DTYPE;
        st = check_norm_gate(ng->gate, in_b, ng->norm_weight, ng->eps, heads, head_dim, o,
                             tokens * heads * head_dim * dtype_size(out_dtype), state_out, st_b);
        if (st != LT_OK) return st;
    }
    if (batch == 0 || heads == 0) return LT_OK;
    if (workspace && workspace_bytes > 0) {
        const Range rw = range_of(workspace, (long long)workspace_bytes);
        if (overlaps(rw, range_of(q, in_b)) || overlaps(rw, range_of(k, in_b)) ||
            overlaps(rw, range_of(v, in_b)) || overlaps(rw, range_of(slopes, heads * 4LL)) ||
            overlaps(rw, range_of(o, tokens * heads * head_dim * dtype_size(out_dtype))) ||
            (state_in && overlaps(rw, range_of(state_in, st_b))) ||
            (state_out && overlaps(rw, range_of(state_out, st_b))) ||
            (ng && (overlaps(rw, range_of(ng->gate, in_b)) ||
                    overlaps(rw, range_of(ng->norm_weight, (long long)heads * head_dim * 4)))))
            return LT_ERR_ALIAS;
    }
    if (tokens == 0 && !state_out) return LT_OK;
    lt::PrefillArgs a{q, k, v, slopes, o, state_in, state_out, nullptr, seqlen, tokens,
                      batch, heads};
    if (ng) a.ng = *ng;
    if (use_scratch) {  // the library's static scratch in place of a workspace
        const hipError_t e =
            lt::noalloc_scratch(static_cast<hipStream_t>(stream), &workspace, &workspace_bytes);
        if (e != hipSuccess) return map_hip(e);
    }
    return launch(a, in_dtype, out_dtype, false, workspace, workspace_bytes, stream, use_scratch);
}

lt_status varlen_impl(const void *q, const void *k, const void *v, lt_dtype in_dtype,
                      const int *cu_seqlens, int num_seqs, long long total_tokens,
                      long long max_seqlen, const float *slopes, void *o, lt_dtype out_dtype,
                      const float *state_in, float *state_out, int heads, int head_dim, int block,
                      void *workspace, size_t workspace_bytes, void *stream,
                      const lt::NormGate *ng) {
    if (num_seqs < 0 || total_tokens < 0) return LT_ERR_SHAPE;
    if (total_tokens > 0x7fffffffLL) return LT_ERR_SHAPE;  // int32 sequence boundaries
    if (max_seqlen < 0 || max_seqlen > total_tokens) return LT_ERR_SHAPE;
    if (max_seqlen == 0) max_seqlen = total_tokens;  // unknown: no sequence is longer
    lt_status st = check_prefill(q, k, v, in_dtype, slopes, o, out_dtype, state_in, state_out,
                                 num_seqs, total_tokens, heads, head_dim, block);
    if (st != LT_OK) return st;
    if (ng) {
        if (in_dtype != LT_BF16) return LT_ERR_DTYPE;
        st = check_norm_gate(ng->gate, total_tokens * heads * head_dim * dtype_size(in_dtype),
                             ng->norm_weight, ng->eps, heads, head_dim, o,
                             total_tokens * heads * head_dim * dtype_size(out_dtype), state_out,
                             (long long)num_seqs * heads * head_dim * head_dim * 4);
        if (st != LT_OK) return st;
    }
    if (num_seqs == 0 || heads == 0) return LT_OK;
    if (!cu_seqlens) return LT_ERR_NULL;
    const long long in_b = total_tokens * heads * head_dim * dtype_size(in_dtype);
    const long long out_b = total_tokens * heads * head_dim * dtype_size(out_dtype);
    const long long st_b = (long long)num_seqs * heads * head_dim * head_dim * 4;
    const Range rcu = range_of(cu_seqlens, (long long)(num_seqs + 1) * 4);
    if (overlaps(rcu, range_of(o, out_b)) || (state_out && overlaps(rcu, range_of(state_out, st_b))))
        return LT_ERR_ALIAS;
    if (workspace && workspace_bytes > 0) {
        const Range rw = range_of(workspace, (long long)workspace_bytes);
        if (overlaps(rw, range_of(q, in_b)) || overlaps(rw, range_of(k, in_b)) ||
            overlaps(rw, range_of(v, in_b)) || overlaps(rw, range_of(slopes, heads * 4LL)) ||
            overlaps(rw, range_of(o, out_b)) || overlaps(rw, rcu) ||
            (state_in && overlaps(rw, range_of(state_in, st_b))) ||
            (state_out && overlaps(rw, range_of(state_out, st_b))) ||
            (ng && (overlaps(rw, range_of(ng->gate, in_b)) ||
                    overlaps(rw, range_of(ng->norm_weight, (long long)heads * head_dim * 4)))))
            return LT_ERR_ALIAS;
    }
    if (total_tokens == 0 && !state_out) return LT_OK;
    // seqlen carries the longest sequence's length (the plan's upper bound)
    lt::PrefillArgs a{q, k, v, slopes, o, state_in, state_out, cu_seqlens, max_seqlen, total_tokens,
                      num_seqs, heads};
    if (ng) a.ng = *ng;
    return launch(a, in_dtype, out_dtype, true, workspace, workspace_bytes, stream);
}

// Decode. With slot_ids, `state` is a pool of num_slots entries of
// [heads, d, d] and sequence b uses entry slot_ids[b] (ids are read on the
// device only; out-of-range ids are padding rows).
lt_status decode_impl(const void *q, const void *k, const void *v, lt_dtype in_dtype,
                      const float *slopes, float *state, void *o, lt_dtype out_dtype, int batch,
                      int heads, int head_dim, void *stream, const lt::NormGate *ng,
                      const int *slot_ids = nullptr, int num_slots = -1) {
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return LT_ERR_DTYPE;
    if (head_dim != lt::kHeadDim || heads < 0 || heads > LT_MAX_HEADS || batch < 0)
        return LT_ERR_SHAPE;
    const bool slots = num_slots >= 0;
    long long units = (long long)batch * heads;
    if (units > 0x7fffffffLL) return LT_ERR_SHAPE;
    long long pool_units = units;
    if (slots && __builtin_mul_overflow((long long)num_slots, (long long)heads, &pool_units))
        return LT_ERR_SHAPE;
    if (pool_units > 0x7fffffffLL) return LT_ERR_SHAPE;
    const long long in_bytes = units * head_dim * dtype_size(in_dtype);
    const long long out_bytes = units * head_dim * dtype_size(out_dtype);
    const long long st_bytes = pool_units * head_dim * head_dim * 4;
    if (ng) {
        const lt_status st = check_norm_gate(ng->gate, in_bytes, ng->norm_weight, ng->eps, heads,
                                             head_dim, o, out_bytes, state, st_bytes);
        if (st != LT_OK) return st;
    }
    if (batch == 0 || heads == 0) return LT_OK;
    if (!q || !k || !v || !slopes || !o || (!state && pool_units > 0) || (slots && !slot_ids))
        return LT_ERR_NULL;
    const Range rq = range_of(q, in_bytes), rk = range_of(k, in_bytes),
                rv = range_of(v, in_bytes), ro = range_of(o, out_bytes),
                rs = range_of(slopes, (long long)heads * 4), rst = range_of(state, st_bytes),
                rid = range_of(slot_ids, slots ? (long long)batch * 4 : 0);
    if (overlaps(ro, rq) || overlaps(ro, rk) || overlaps(ro, rv) || overlaps(ro, rs) ||
        overlaps(ro, rst) || overlaps(rst, rq) || overlaps(rst, rk) || overlaps(rst, rv) ||
        overlaps(rst, rs) || overlaps(ro, rid) || overlaps(rst, rid))
        return LT_ERR_ALIAS;
    lt::DecodeArgs a{q, k, v, slopes, state, o, batch, heads};
    a.seq_stride = decode_seq_stride(batch);
    if (ng) a.ng = *ng;
    if (slots) {
        a.slot_ids = slot_ids;
        a.num_slots = num_slots;
    }
    return map_hip(lt::launch_decode(a, in_dtype, out_dtype, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

LT_API lt_status lt_prefill(const void *q, const void *k, const void *v, lt_dtype in_dtype,
                            const float *slopes, void *o, lt_dtype out_dtype,
                            const float *state_in, float *state_out,
                            int batch, long long seqlen, int heads, int head_dim, int block,
                            void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_impl(q, k, v, in_dtype, slopes, o, out_dtype, state_in, state_out, batch, seqlen,
                        heads, head_dim, block, workspace, workspace_bytes, stream, nullptr);
}

LT_API lt_status lt_prefill_noalloc(const void *q, const void *k, const void *v,
                                    lt_dtype in_dtype, const float *slopes, void *o,
                                    lt_dtype out_dtype, const float *state_in, float *state_out,
                                    int batch, long long seqlen, int heads, int head_dim, int block,
                                    void *stream) {
    return prefill_impl(q, k, v, in_dtype, slopes, o, out_dtype, state_in, state_out, batch, seqlen,
                        heads, head_dim, block, nullptr, 0, stream, nullptr, true);
}

LT_API lt_status lt_prefill_norm_gate(const void *q, const void *k, const void *v,
                                      lt_dtype in_dtype, const float *slopes, const void *gate,
                                      const float *norm_weight, float eps, void *y,
                                      lt_dtype out_dtype, const float *state_in, float *state_out,
                                      int batch, long long seqlen, int heads, int head_dim,
                                      int block, void *workspace, size_t workspace_bytes,
                                      void *stream) {
    const lt::NormGate ng{gate, norm_weight, eps};
    return prefill_impl(q, k, v, in_dtype, slopes, y, out_dtype, state_in, state_out, batch, seqlen,
                        heads, head_dim, block, workspace, workspace_bytes, stream, &ng);
}

LT_API lt_status lt_prefill_varlen(const void *q, const void *k, const void *v, lt_dtype in_dtype,
                                   const int *cu_seqlens, int num_seqs, long long total_tokens,
                                   long long max_seqlen, const float *slopes, void *o,
                                   lt_dtype out_dtype, const float *state_in, float *state_out,
                                   int heads, int head_dim, int block, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    return varlen_impl(q, k, v, in_dtype, cu_seqlens, num_seqs, total_tokens, max_seqlen, slopes, o,
                       out_dtype, state_in, state_out, heads, head_dim, block, workspace,
                       workspace_bytes, stream, nullptr);
}

LT_API lt_status lt_prefill_varlen_norm_gate(const void *q, const void *k, const void *v,
                                             lt_dtype in_dtype, const int *cu_seqlens,
                                             int num_seqs, long long total_tokens,
                                             long long max_seqlen, const float *slopes,
                                             const void *gate, const float *norm_weight, float eps,
                                             void *y, lt_dtype out_dtype, const float *state_in,
                                             float *state_out, int heads, int head_dim, int block,
                                             void *workspace, size_t workspace_bytes,
                                             void *stream) {
    const lt::NormGate ng{gate, norm_weight, eps};
    return varlen_impl(q, k, v, in_dtype, cu_seqlens, num_seqs, total_tokens, max_seqlen, slopes, y,
                       out_dtype, state_in, state_out, heads, head_dim, block, workspace,
                       workspace_bytes, stream, &ng);
}

LT_API lt_status lt_decode(const void *q, const void *k, const void *v, lt_dtype in_dtype,
                           const float *slopes, float *state, void *o, lt_dtype out_dtype,
                           int batch, int heads, int head_dim, void *stream) {
    return decode_impl(q, k, v, in_dtype, slopes, state, o, out_dtype, batch, heads, head_dim,
                       stream, nullptr);
}

LT_API lt_status lt_prefill_backward(const void *q, const void *k, const void *v, const void *dout,
                                     lt_dtype in_dtype, const float *slopes, const float *state_in,
                                     const float *d_state_out, void *dq, void *dk, void *dv,
                                     lt_dtype grad_dtype, float *d_state_in, int batch,
                                     long long seqlen, int heads, int head_dim, int block,
                                     void *workspace, size_t workspace_bytes, void *stream) {
    if (!dtype_ok(in_dtype) || !dtype_ok(grad_dtype)) return LT_ERR_DTYPE;
    if (in_dtype != LT_BF16) return LT_ERR_DTYPE;
    if (batch < 0 || seqlen < 0 || head_dim != lt::kHeadDim || heads < 0 || heads > LT_MAX_HEADS)
        return LT_ERR_SHAPE;
    if (block < 1 || block > LT_MAX_BLOCK) return LT_ERR_BLOCK;
    long long tokens, in_b, g_b, st_b, grid;
    if (__builtin_mul_overflow((long long)batch, seqlen, &tokens) ||
        !mul4(tokens, heads, head_dim, 2, &in_b) ||
        !mul4(tokens, heads, head_dim, dtype_size(grad_dtype), &g_b) ||
        !mul4(batch, heads, (long long)head_dim * head_dim, 4, &st_b) ||
        !mul4(batch, heads, lt::kValueSlices, 1, &grid) || grid > 0x7fffffffLL)
        return LT_ERR_SHAPE;
    if (batch == 0 || heads == 0) return LT_OK;
    if (!slopes) return LT_ERR_NULL;
    if (tokens > 0 && (!q || !k || !v || !dout || !dq || !dk || !dv)) return LT_ERR_NULL;
    const Range ins[] = {range_of(q, in_b), range_of(k, in_b), range_of(v, in_b),
                         range_of(dout, in_b), range_of(slopes, heads * 4LL),
                         range_of(state_in, state_in ? st_b : 0),
                         range_of(d_state_out, d_state_out ? st_b : 0)};
    const Range outs[] = {range_of(dq, g_b), range_of(dk, g_b), range_of(dv, g_b),
                          range_of(d_state_in, d_state_in ? st_b : 0),
                          range_of(workspace, workspace ? (long long)workspace_bytes : 0)};
    for (const Range &o : outs) {
        for (const Range &i : ins)
            if (overlaps(o, i)) return LT_ERR_ALIAS;
    }
    for (int x = 0; x < 5; ++x)
        for (int y = x + 1; y < 5; ++y)
            if (overlaps(outs[x], outs[y])) return LT_ERR_ALIAS;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (tokens > 0) {
        // dQ = forward(dO, V, K) carrying S_0^T
        lt::PrefillArgs a{dout, v, k, slopes, dq, state_in, nullptr, nullptr, seqlen, tokens,
                          batch, heads};
        a.state_in_t = true;
        const lt_status s1 = launch(a, LT_BF16, grad_dtype, false, workspace, workspace_bytes, stream);
        if (s1 != LT_OK) return s1;
    }
    if (tokens == 0 && !d_state_in) return LT_OK;
    const lt::BackwardArgs b{q, k, v, dout, slopes, d_state_out, dk, dv, d_state_in, seqlen,
                             batch, heads};
    // the reverse pass splits long sequences like the forward when the
    // workspace allows (the dq pass above has finished with it by then)
    lt::PrefillPlan p = lt::plan_prefill(batch, seqlen, heads, LT_BF16, false, kPrepassWide,
                                         workspace ? workspace_bytes : 0);
    if (p.value_slices != 1) {
        p = lt::PrefillPlan{};
        p.seg_len = seqlen;
    }
    return map_hip(lt::launch_backward_kv(b, p, workspace, grad_dtype, st));
}

LT_API lt_status lt_decode_slots(const void *q, const void *k, const void *v, lt_dtype in_dtype,
                                 const float *slopes, float *state_pool, int num_slots,
                                 const int *slot_ids, void *o, lt_dtype out_dtype, int batch,
                                 int heads, int head_dim, void *stream) {
    if (num_slots < 0) return LT_ERR_SHAPE;
    return decode_impl(q, k, v, in_dtype, slopes, state_pool, o, out_dtype, batch, heads, head_dim,
                       stream, nullptr, slot_ids, num_slots);
}

LT_API lt_status lt_decode_norm_gate(const void *q, const void *k, const void *v,
                                     lt_dtype in_dtype, const float *slopes, float *state,
                                     const void *gate, const float *norm_weight, float eps,
                                     void *y, lt_dtype out_dtype, int batch, int heads,
                                     int head_dim, void *stream) {
    const lt::NormGate ng{gate, norm_weight, eps};
    return decode_impl(q, k, v, in_dtype, slopes, state, y, out_dtype, batch, heads, head_dim,
                       stream, &ng);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Softmax attention (grouped K/V heads, partial RoPE)

namespace {

lt_status check_softmax_common(int q_heads, int kv_heads, int head_dim, int rope_dims,
                               double rope_base, float scale) {
    if (head_dim != lt::kHeadDim || q_heads < 0 || kv_heads < 0 || q_heads > LT_MAX_HEADS ||
        kv_heads > LT_MAX_HEADS)
        return LT_ERR_SHAPE;
    if ((q_heads == 0) != (kv_heads == 0)) return LT_ERR_SHAPE;
    if (kv_heads > 0 && q_heads % kv_heads != 0) return LT_ERR_SHAPE;
    if (rope_dims < 0 || rope_dims > head_dim || rope_dims % 32 != 0) return LT_ERR_SHAPE;
    if (!(rope_base > 1.0) || rope_base > 1e300) return LT_ERR_VALUE;
    if (!(scale > 0.f) || scale > 3.0e38f) return LT_ERR_VALUE;
    return LT_OK;
}

}  // namespace

extern "C" {

LT_API lt_status lt_softmax_prefill(const void *q, const void *k, const void *v, void *o,
                                    lt_dtype out_dtype, void *k_rope, int batch, long long seqlen,
                                    int q_heads, int kv_heads, int head_dim, int rope_dims,
                                    double rope_base, float scale, long long pos0, void *stream) {
    if (!dtype_ok(out_dtype)) return LT_ERR_DTYPE;
    if (batch < 0 || seqlen < 0 || pos0 < 0) return LT_ERR_SHAPE;
    const lt_status c = check_softmax_common(q_heads, kv_heads, head_dim, rope_dims, rope_base, scale);
    if (c != LT_OK) return c;
    long long tokens, q_b, kv_b, o_b, grid, last_pos;
    if (__builtin_mul_overflow((long long)batch, seqlen, &tokens) ||
        !mul4(tokens, q_heads, head_dim, 2, &q_b) || !mul4(tokens, kv_heads, head_dim, 2, &kv_b) ||
        !mul4(tokens, q_heads, head_dim, dtype_size(out_dtype), &o_b) ||
        !mul4((seqlen + 127) / 128, batch, q_heads, 1, &grid) || grid > 0x7fffffffLL ||
        __builtin_add_overflow(pos0, seqlen, &last_pos) ||
        (long long)kv_heads * head_dim * 64 > 0x7fffffffLL)
        return LT_ERR_SHAPE;
    if (tokens == 0 || q_heads == 0) return LT_OK;
    if (!q || !k || !v || !o || !k_rope) return LT_ERR_NULL;
    const Range ins[] = {range_of(q, q_b), range_of(k, kv_b), range_of(v, kv_b)};
    const Range outs[] = {range_of(o, o_b), range_of(k_rope, kv_b)};
    for (const Range &x : outs)
        for (const Range &i : ins)
            if (overlaps(x, i)) return LT_ERR_ALIAS;
    if (overlaps(outs[0], outs[1])) return LT_ERR_ALIAS;
    lt::SoftmaxArgs a{q, k, v, o, batch, seqlen, pos0, q_heads, kv_heads, rope_dims,
                      __builtin_log2(rope_base), scale};
    return map_hip(lt::launch_softmax_prefill(a, k_rope, out_dtype, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Waves a softmax decode launch should reach: eight per CU keeps enough
// cache reads in flight to cover HBM latency.
constexpr long long kDecodeWaves = 2048;
// Fewest keys worth a split of their own.
constexpr long long kMinDecodeChunk = 256;

// Splits are planned on the capacity (the lengths live on the device): each
// (sequence, K/V head) gets `splits` waves of `chunk` keys; splits that start
// past a sequence's length exit at once.
lt::SoftmaxDecodePlan plan_softmax_decode(int batch, long long capacity, int kv_heads) {
    lt::SoftmaxDecodePlan p;
    const long long units = (long long)batch * kv_heads;
    long long splits = (kDecodeWaves + units - 1) / units;
    const long long max_splits = (capacity + kMinDecodeChunk - 1) / kMinDecodeChunk;
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    long long chunk = (capacity + splits - 1) / splits;
    chunk = (chunk + 31) / 32 * 32;
    p.chunk = chunk;
    p.splits = (int)((capacity + chunk - 1) / chunk);
    return p;
}

lt_status check_softmax_decode(int batch, long long capacity, int q_heads, int kv_heads,
                               int head_dim, long long *tokens_out) {
    if (batch < 0 || capacity < 0 || capacity > 0x7fffffffLL || head_dim != lt::kHeadDim)
        return LT_ERR_SHAPE;
    if (kv_heads > 0 && q_heads / kv_heads > 32) return LT_ERR_SHAPE;
    long long tokens;
    if (__builtin_mul_overflow((long long)batch, capacity, &tokens)) return LT_ERR_SHAPE;
    *tokens_out = tokens;
    return LT_OK;
}

}  // namespace

extern "C" {

LT_API size_t lt_softmax_decode_workspace_bytes(int batch, long long capacity, int q_heads,
                                                int kv_heads, int head_dim) {
    long long tokens;
    if (batch <= 0 || capacity <= 0 || q_heads <= 0 || kv_heads <= 0 || q_heads > LT_MAX_HEADS ||
        q_heads % kv_heads != 0 ||
        check_softmax_decode(batch, capacity, q_heads, kv_heads, head_dim, &tokens) != LT_OK)
        return 0;
    const lt::SoftmaxDecodePlan p = plan_softmax_decode(batch, capacity, kv_heads);
    return (size_t)lt::softmax_decode_workspace(batch, q_heads, p.splits);
}

LT_API lt_status lt_softmax_decode(const void *q, const void *k_new, const void *v_new,
                                   void *k_cache, void *v_cache, const int *lengths, void *o,
                                   lt_dtype out_dtype, int batch, long long capacity, int q_heads,
                                   int kv_heads, int head_dim, int rope_dims, double rope_base,
                                   float scale, void *workspace, size_t workspace_bytes,
                                   void *stream) {
    if (!dtype_ok(out_dtype)) return LT_ERR_DTYPE;
    const lt_status c = check_softmax_common(q_heads, kv_heads, head_dim, rope_dims, rope_base, scale);
    if (c != LT_OK) return c;
    long long tokens;
    const lt_status c2 = check_softmax_decode(batch, capacity, q_heads, kv_heads, head_dim, &tokens);
    if (c2 != LT_OK) return c2;
    long long q_b, kv_b, cache_b, o_b, waves;
    if (!mul4(batch, q_heads, head_dim, 2, &q_b) || !mul4(batch, kv_heads, head_dim, 2, &kv_b) ||
        !mul4(tokens, kv_heads, head_dim, 2, &cache_b) ||
        !mul4(batch, q_heads, head_dim, dtype_size(out_dtype), &o_b) ||
        !mul4(batch, kv_heads, 1, 1, &waves) || waves > 0x7fffffffLL / 64 ||
        (long long)batch * q_heads > 0x7fffffffLL)
        return LT_ERR_SHAPE;
    if (batch == 0 || q_heads == 0) return LT_OK;
    if (capacity == 0) return LT_ERR_SHAPE;  // no room for the new token
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !lengths || !o) return LT_ERR_NULL;
    lt::SoftmaxDecodePlan p = plan_softmax_decode(batch, capacity, kv_heads);
    const long long ws_need = lt::softmax_decode_workspace(batch, q_heads, p.splits);
    const bool use_ws = ws_need > 0 && workspace && (long long)workspace_bytes >= ws_need;
    if (!use_ws) {
        p.splits = 1;
        p.chunk = (capacity + 31) / 32 * 32;
    }
    const Range ins[] = {range_of(q, q_b), range_of(k_new, kv_b), range_of(v_new, kv_b),
                         range_of(lengths, batch * 4LL)};
    const Range outs[] = {range_of(o, o_b), range_of(k_cache, cache_b), range_of(v_cache, cache_b),
                          range_of(workspace, use_ws ? ws_need : 0)};
    for (const Range &x : outs)
        for (const Range &i : ins)
            if (overlaps(x, i)) return LT_ERR_ALIAS;
    for (int x = 0; x < 4; ++x)
        for (int y = x + 1; y < 4; ++y)
            if (overlaps(outs[x], outs[y])) return LT_ERR_ALIAS;
    const lt::SoftmaxDecodeArgs a{q, k_new, v_new, k_cache, v_cache, lengths, o, batch, capacity,
                                  q_heads, kv_heads, rope_dims, __builtin_log2(rope_base), scale};
    return map_hip(lt::launch_softmax_decode(a, p, use_ws ? static_cast<float *>(workspace) : nullptr,
                                             out_dtype, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
