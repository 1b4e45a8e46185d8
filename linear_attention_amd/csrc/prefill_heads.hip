// Lightning Attention prefill for bf16 inputs on gfx950 (MI355X): one 8-wave
// workgroup per (sequence, head, segment of the sequence).
//
// Operator (MiniMax Signal Lab · M1, §03 Lightning Attention), per head with a
// d x d fp32 state S carried across blocks of m tokens (positions 1..m):
//   O_t = [(Q_t K_t^T) ⊙ D] V_t + (Q_t ⊙ d_q) S_{t-1}
//   S_t = e^{-s m} S_{t-1} + (K_t ⊙ d_k)^T V_t
//   D_ij = e^{-s(i-j)}[i>=j],  d_q[i] = e^{-s i},  d_k[j] = e^{-s(m-j)}.
// The result does not depend on the block length, so the kernel walks each
// sequence in 64-token sub-blocks.
//
// gfx950 design:
//  * A workgroup owns a whole head (all 128 value columns), so the 64x64 score
//    tile of a sub-block is computed once, and one loop iteration moves 80 KiB
//    of HBM traffic (q, k, v in bf16, o in fp32) against ~44 MFMA issue slots
//    per SIMD. Eight waves give two waves per SIMD to hide latency.
//  * All products use v_mfma_f32_32x32x16_bf16 (fp32 accumulation). Wave w owns
//    output block (queries 32*(w/4).., value columns 32*(w%4)..) and state
//    blocks (keys 64*(w/4).., the same 32 columns); waves 0..2 also compute the
//    three causal 32x32 score blocks and share P through LDS.
//  * Q, K, V stay row-major in LDS. The transposed operands (V^T for P V, K^T
//    and (V ⊙ d_k)^T for the state update) are read with ds_read_b64_tr_b16,
//    which returns a 4x16 block transposed across each 16-lane group, so no
//    VALU transposes are needed. Only V ⊙ d_k is formed by VALU.
//  * The state lives in the MFMA accumulators of the eight waves for the whole
//    segment; each sub-block it is also written to LDS once as bf16 S^T, the
//    operand of the next sub-block's inter-block product.
//  * Batch-1 prefill has only 64 (sequence, head) pairs for 256 CUs, so long
//    sequences are cut into segments. A pre-pass kernel computes the state
//    contributed by fixed pieces of every segment but the last (the same state
//    update without outputs) into a workspace; segment g starts from
//    e^{-s*start_g} S_0 plus each piece's state decayed to start_g.
//  * Heads whose decay ends their memory well within a segment (below 2^-16
//    after W tokens, W < the segment length) skip the pre-pass. Their tokens
//    are cut into ranges of equal cost, one per remaining workgroup, and a
//    range that starts at token t0 > 0 first rebuilds its carried-in state
//    from the W tokens before t0 by state-only steps. A small finishing pass
//    restores the NaN and Inf that the exact operator carries past a range's
//    end (a warm-up window cannot see them).
//  * Outputs go through LDS and leave as whole rows (full 512-byte fp32 rows
//    stream far better than the 32-byte pieces of the accumulator layout).
//  * Shared building blocks (layouts, operand loads, staging, state update)
//    are in tiles.h.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "internal.h"
#include "tiles.h"

namespace lt {
namespace {

// Rows [0, m) of the staged tile with the post-sum normalisation and gate:
// y = o / sqrt(mean(o^2) + eps) * w * sigmoid(g). Thread layout as the fp32
// store_rows (rows (tid/32) + 16j, columns 4(tid%32)..+3). Each row's sum of
// squares comes from rss[row][0..3], the partial sums of its four 32-column
// blocks that the waves wrote from their accumulators (row_sumsq). gr[j] holds
// the four bf16 gate values of row j, w the four weights of the thread's columns.
__device__ __forceinline__ void put4(float *p, float4 y) { stream_store(p, y); }
__device__ __forceinline__ void put4(__bf16 *p, float4 y) {
    const bf16x4 b = {static_cast<__bf16>(y.x), static_cast<__bf16>(y.y), static_cast<__bf16>(y.z),
                      static_cast<__bf16>(y.w)};
    stream_store_bits(p, b);
}
__device__ __forceinline__ float sigmoid(float g) {
    return __builtin_amdgcn_rcpf(1.f + fast_exp2(-g * LOG2E));
}

// The wave's output block holds, per lane, 16 of the 32 columns (value block
// 32cq..) of query row 32qh + lane%32; lanes l and l^32 hold the other 16.
__device__ __forceinline__ void row_sumsq(float *rss, const f32x16 &o, int qh, int cq, int lane) {
    float ss = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) ss += o[v] * o[v];
    ss += __shfl_xor(ss, 32);
    if (lane < 32) rss[(32 * qh + lane) * 4 + cq] = ss;
}

template <bool FULL, typename OutT>
__device__ __forceinline__ void store_rows_norm_gate(OutT *out, long long ts, const float *Os,
                                                     const float *rss, int m, int tid,
                                                     const uint2 (&gr)[4], float4 w, float eps) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = (tid >> 5) + 16 * j, col = 4 * (tid & 31);
        const float4 x = *reinterpret_cast<const float4 *>(Os + ooff(row, col));
        const float4 p = *reinterpret_cast<const float4 *>(rss + 4 * row);
        const float inv = __builtin_amdgcn_rsqf((p.x + p.y + p.z + p.w) * (1.f / D) + eps);
        const float g0 = __uint_as_float(gr[j].x << 16), g1 = __uint_as_float(gr[j].x & 0xffff0000u);
        const float g2 = __uint_as_float(gr[j].y << 16), g3 = __uint_as_float(gr[j].y & 0xffff0000u);
        const float f0 = inv * w.x * sigmoid(g0), f1 = inv * w.y * sigmoid(g1);
        const float f2 = inv * w.z * sigmoid(g2), f3 = inv * w.w * sigmoid(g3);
        const float4 y = make_float4(x.x * f0, x.y * f1, x.z * f2, x.w * f3);
        if (FULL || row < m) put4(out + row * ts + col, y);
    }
}

// Pre-pass: workgroup (unit, head, piece j) runs the state update over the
// full 64-token sub-blocks of its group of pieces without outputs, writing its
// state and, if a segment boundary falls strictly inside the group, B_g on the
// way. Workgroup b < units * heads first resets the records of pair b if that
// pair takes warm-up ranges.
__global__ __launch_bounds__(NT, 2) void piece_state_kernel(PrefillArgs a, Segmented sp, float *ws) {
    __shared__ __attribute__((aligned(16))) __bf16 Ks[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Vds[C * D];
    __shared__ short heads_pre[kMaxPairs], heads_warm[kMaxPairs];

    if ((int)blockIdx.x < a.units * a.heads && !takes_prepass(sp, a.slopes[blockIdx.x % a.heads] * LOG2E))
        reset_records(warm_records(sp, ws, blockIdx.x), NT);

    // workgroup b takes group b % gph of the (b / gph)-th pre-pass pair (in
    // (unit, head) order), gph groups of kgr pieces per pair; the working
    // workgroups are the first units * npre * gph (at most kPrepassActive +
    // units * heads: the launch is sized for that), which the hardware spreads
    // over all XCDs. The group's state goes to the slot of its last piece.
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Routes rt = split_heads(a.slopes, a.heads, sp, heads_pre, heads_warm, w == 0);
    if (rt.npre == 0) return;  // every head on warm-up segments: no pre-pass
    const int kgr = prepass_group_of(rt.npre, a.units, sp);
    const int gph = (sp.pieces + kgr - 1) / kgr;
    if ((int)blockIdx.x >= a.units * rt.npre * gph) return;
    __syncthreads();  // wave 0's head lists are visible
    const int j = (blockIdx.x % gph) * kgr;
    const int i = blockIdx.x / gph;
    const int n = i / rt.npre, h = heads_pre[i % rt.npre];
    const int uh = n * a.heads + h;
    const int qh = w >> 2, cq = w & 3, r32 = lane & 31, hf = lane >> 5;

    const float s2 = a.slopes[h] * LOG2E;
    const int jl = j + kgr - 1 < sp.pieces - 1 ? j + kgr - 1 : sp.pieces - 1;
    const SeqRange sr = sequence_of(a, n);
    const long long covered = sp.covered(sr.len);
    const long long t0 = j * sp.piece_len;
    if (t0 >= covered) return;  // past this sequence's pre-pass tokens
    const long long t1 = t0 + kgr * sp.piece_len < covered ? t0 + kgr * sp.piece_len : covered;
    const int ts = a.heads * D;
    const long long base = ((sr.start + t0) * a.heads + h) * (long long)D;
    const uint16_t *kg = static_cast<const uint16_t *>(a.k) + base;
    const uint16_t *vg = static_cast<const uint16_t *>(a.v) + base;
    float *u = sp.unit(ws, uh);

    f32x16 S[2];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) S[db][v] = 0.f;
    // Writes S to workspace slot `slot` of this (unit, head). The empty asm
    // keeps the compiler from computing the addresses of both stores before
    // the loops (which costs ~50 registers and spills).
    auto store_state = [&](int slot) {
        asm volatile("" : "+s"(slot));
        float *dst = Segmented::slot(u, slot);
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                dst[(64 * qh + 32 * db + 8 * (v >> 2) + 4 * hf + (v & 3)) * D + 32 * cq + r32] = S[db][v];
    };

    Stage<false> st0, st1;
    const long long nch = (t1 - t0) / C;  // even, >= 2: all full sub-blocks
    const float bd = fast_exp2(-s2 * (float)C);
    auto prefetch = [&](Stage<false> &st, long long c) {
        // past the end one row is read again (row stride 0; ignored), so the
        // count of loads stays fixed without a whole sub-block of traffic
        const bool in = c < nch;
        const long long off = (in ? c : nch - 1) * C * (long long)ts;
        st.load(nullptr, kg + off, vg + off, in ? ts : 0, C, tid);
    };
    auto step = [&](long long c, Stage<false> &st) {
        // Nothing of this sub-block may be scheduled into the previous one:
        // touching its registers there waits for its loads one sub-block early.
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        st.template store<true>(nullptr, Ks, nullptr, Vds, C, s2, tid);
        prefetch(st, c + 2);
        __syncthreads();
        state_update(S, Ks, Vds, bd, qh, cq, lane);
    };
    // sub-blocks [c0, c1), both even; sub-block c is staged in st[c % 2]
    auto run = [&](long long c0, long long c1) {
        for (long long c = c0; c < c1; c += 2) {
            step(c, st0);
            step(c + 1, st1);
        }
    };
    prefetch(st0, 0);
    prefetch(st1, 1);
    // Up to the segment boundary inside the piece (if any: B_g), then the rest.
    // Without one the first part is the whole piece, the second is empty, and
    // P_j is written twice with the same values (a branch around either store
    // costs the loop ~50 registers).
    const int gb = (int)(t0 / sp.seg_len) + 1;  // first segment boundary after t0
    const long long b = gb * sp.seg_len;
    const long long cb = b < t1 ? (b - t0) / C : nch;
    run(0, cb);
    store_state(b < t1 ? sp.partial_slot(gb) : jl);
    run(cb, nch);
    store_state(jl);
}


// ---------------------------------------------------------------------------
constexpr int kRankUnits = 64;

// Warm-up cost of a token against an output token. By bytes a warm-up token
// moves its k and v rows (2 x 256 B) against q, k, v, the output row and, with
// the norm-gate epilogue, the gate row of an output token; the warm-up's steps
// (two barriers per 64-token sub-block, no output stores to overlap) run below
// the streaming rate, by the factor measured on the M1 layer (24-27 ns per
// warm-up token against 53 ns per output token with fp32 outputs).
template <typename OutT, bool NG>
__device__ constexpr double warm_cost() {
    return 1.25 * 512.0 / (768.0 + 128.0 * sizeof(OutT) + (NG ? 256.0 : 0.0));
}

// A workgroup's current piece, as thread 0 lays it out for the others: rows
// of the piece's first token (k and v: of its warm-up's first token; row
// stride ts elements), its length, the carried-in state and where the end
// state goes.
struct Piece {
    const uint16_t *q, *k, *v, *gate;
    void *o;
    const float *nw;    // the head's normalisation weights (norm-gate epilogue)
    const float *s_in;  // carried-in state (nullptr: zero)
    float *dst;         // end == 1: the final state's destination
    int *rec;           // end == 2: the pair's records
    float *u;           // comb_g > 0: the pair's workspace unit
    long long covered;  // comb_g > 0: the pair's pre-pass tokens
    long long len, warm;  // tokens of the piece; warm-up tokens before it (whole sub-blocks)
    float s2, eps;
    int ts;
    int uh;      // -1: no more pieces
    int s_in_t;  // s_in transposed
    int cut;     // end == 2: the token the piece ends at
    int end;     // 0 nothing, 1 the final state to dst, 2 records if the end state is non-finite
    int comb_g;  // > 0: segment comb_g of a pre-pass pair, whose start state the piece combines
    int kg;      // comb_g > 0: pre-pass pieces per group
};
template <typename OutT>
__device__ void piece_rows(Piece &p, const PrefillArgs &a, int n, int h, long long t0, long long t1,
                           long long t0w) {
    const long long start = sequence_of(a, n).start;
    const long long r0 = ((start + t0) * a.heads + h) * (long long)D, rw = ((start + t0w) * a.heads + h) * (long long)D;
    p.q = static_cast<const uint16_t *>(a.q) + r0;
    p.k = static_cast<const uint16_t *>(a.k) + rw;
    p.v = static_cast<const uint16_t *>(a.v) + rw;
    p.o = static_cast<OutT *>(a.o) + r0;
    p.gate = a.ng.gate ? static_cast<const uint16_t *>(a.ng.gate) + r0 : nullptr;
    p.nw = a.ng.norm_weight ? a.ng.norm_weight + h * D : nullptr;
    p.len = t1 - t0;
    p.warm = t0 - t0w;
    p.s2 = a.slopes[h] * LOG2E;
    p.eps = a.ng.eps;
    p.ts = a.heads * D;
    p.uh = n * a.heads + h;
}

// A warm-route piece of pair (n, h): tokens [t0, t1) of a sequence of len.
template <typename OutT>
__device__ void warm_piece(Piece &p, const PrefillArgs &a, const Segmented &sp, float *ws, int n, int h,
                           long long t0, long long t1, long long len) {
    const long long wl = warm_len(a.slopes[h] * LOG2E);
    const long long t0w = t0 > wl ? t0 - wl : 0;
    piece_rows<OutT>(p, a, n, h, t0, t1, t0w);
    const size_t sb = (size_t)p.uh * D * D;
    if (t0w == 0 && a.state_in) {  // the warm-up reaches the sequence start: exact
        p.s_in = a.state_in + sb;
        p.s_in_t = a.state_in_t;
    }
    if (t1 < len) {
        p.rec = warm_records(sp, ws, p.uh);
        p.cut = (int)t1;
        p.end = 2;
    } else if (a.state_out) {
        // on in-place calls other pieces of the pair may still read S_0
        p.dst = a.state_in == a.state_out ? sp.final_state(sp.unit(ws, p.uh)) : a.state_out + sb;
        p.end = 1;
    }
}

// The next piece of this workgroup (thread 0; the arguments are LDS copies,
// so that none of them stays in registers through a piece).
template <typename OutT>
__device__ Piece next_piece(const PrefillArgs &a, const Segmented &sp, float *ws, int mode, int k,
                            PlanState &ps, const short *heads_pre, const short *heads_warm, const double *cpre,
                            const long long *bulk, const short *qlist, const int *by_rank) {
    const PieceRange r = next_range(SeqLens{a.cu_seqlens, a.total_tokens, a.seqlen}, a.heads, sp, mode, k, ps,
                                    heads_pre, heads_warm, cpre, bulk, qlist,
                                    a.cu_seqlens && a.units <= kRankUnits ? by_rank : nullptr);
    Piece p{};
    p.uh = -1;
    if (r.n < 0) return p;
    if (r.kind == 0) {  // the whole sequence of one pair
        piece_rows<OutT>(p, a, r.n, r.h, 0, r.len, 0);
        const size_t sb = (size_t)p.uh * D * D;
        p.s_in = a.state_in ? a.state_in + sb : nullptr;
        p.s_in_t = a.state_in_t;
        p.dst = a.state_out ? a.state_out + sb : nullptr;
        p.end = p.dst ? 1 : 0;
    } else if (r.kind == 1) {  // one segment of a pre-pass pair: S_0, then the combine of the pieces before it
        piece_rows<OutT>(p, a, r.n, r.h, r.t0, r.t1, r.t0);
        const size_t sb = (size_t)p.uh * D * D;
        float *u = sp.unit(ws, p.uh);
        p.s_in = a.state_in ? a.state_in + sb : nullptr;
        p.s_in_t = a.state_in_t;
        p.u = u;
        p.comb_g = r.g;
        p.kg = prepass_group_of(ps.npre, a.units, sp);
        p.covered = sp.covered(r.len);
        if (a.state_out && r.g == sp.used(r.len) - 1) {
            // on in-place calls the pair's other segments may still read S_0
            p.dst = a.state_in == a.state_out ? sp.final_state(u) : a.state_out + sb;
            p.end = 1;
        }
    } else {
        warm_piece<OutT>(p, a, sp, ws, r.n, r.h, r.t0, r.t1, r.len);
    }
    return p;
}

template <typename OutT, bool NG>
__global__ __launch_bounds__(NT) void head_kernel(PrefillArgs a, Segmented sp, float *ws) {
    __shared__ __attribute__((aligned(16))) __bf16 Qs[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Ks[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Vs[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Vds[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Sts[2][D * D];
    __shared__ __attribute__((aligned(16))) __bf16 Ps[C * PW];
    __shared__ __attribute__((aligned(16))) float Wn[NG ? D : 1];
    __shared__ __attribute__((aligned(16))) float Rss[NG ? C * 4 : 1];  // per-row partial sums of o^2
    __shared__ double cpre[kMaxPairs + 1];
    __shared__ long long bulk[kMaxPairs];
    __shared__ short qlist[kMaxPairs];  // pairs that give fine chunks
    __shared__ int fq[2];               // their count, chunks per pair
    __shared__ short heads_pre[kMaxPairs], heads_warm[kMaxPairs];
    __shared__ int by_rank[kRankUnits];
    __shared__ long long rlen[kRankUnits];
    __shared__ PlanState ps;
    __shared__ Piece pc;
    __shared__ __attribute__((aligned(16))) unsigned char args_lds[sizeof(PrefillArgs)];
    __shared__ __attribute__((aligned(16))) unsigned char sp_lds[sizeof(Segmented)];
    __shared__ float *ws_lds;

    const int segments = sp.segments;
    // thread indices of the set-up (each piece recomputes its own, below)
    const int t0id = threadIdx.x, lane0 = t0id & 63;
    const int w = __builtin_amdgcn_readfirstlane(t0id >> 6);
    const SeqLens lens{a.cu_seqlens, a.total_tokens, a.seqlen};
    if (t0id == 0) {
        *reinterpret_cast<PrefillArgs *>(args_lds) = a;
        *reinterpret_cast<Segmented *>(sp_lds) = sp;
        ws_lds = ws;
    }

    // ---- this workgroup's work: pieces (pair uh, tokens [t0, t1)), each
    // starting from S_0 (combined with the pre-pass's states of the earlier
    // tokens on the pre-pass route), zero, and a warm-up
    int mode;  // 0: one pair, whole (no segments); 1: one pre-pass segment; 2: warm ranges
    if (segments == 1) {
        mode = 0;
        // Packed batches of up to kRankUnits sequences run their longest
        // sequences first: unit slot r takes the sequence of rank r by length
        // (descending, ties by index), so the long whole-sequence workgroups do
        // not start last and leave the end of the launch to a few CUs.
        if (a.cu_seqlens && a.units <= kRankUnits) {
            if (t0id < a.units) rlen[t0id] = lens.len(t0id);
            __syncthreads();
            if (t0id < a.units) {
                const long long li = rlen[t0id];
                int r = 0;
                for (int j = 0; j < a.units; ++j) r += rlen[j] > li || (rlen[j] == li && j < t0id);
                by_rank[r] = t0id;
            }
        }
    } else {
        const Routes rt = split_heads(a.slopes, a.heads, sp, heads_pre, heads_warm, w == 0);
        __syncthreads();  // wave 0's head lists are visible
        const long long pre_wgs = (long long)a.units * rt.npre * segments;
        mode = (long long)blockIdx.x < pre_wgs ? 1 : 2;
        const int pw = a.units * rt.nwarm;  // warm pairs
        if (mode == 2 && w == 0)
            warm_plan(lens, a.slopes, heads_warm, rt.nwarm, pw, (double)pw * segments, warm_cost<OutT, NG>(), kFineChunk,
                      cpre, bulk, qlist, fq);
        __syncthreads();  // cpre, bulk, qlist and fq are visible
        if (t0id == 0) {
            ps.npre = rt.npre;
            ps.nwarm = rt.nwarm;
            ps.pw = pw;
            if (mode == 2)
                warm_plan_state(ps, cpre, fq, pw, segments, (int)((long long)blockIdx.x - pre_wgs), kFineChunk,
                                warm_records(sp, ws, heads_warm[0]) + kFineCounter);  // in the first warm pair's records
        }
    }

    // ---- the pieces
    f32x16 S[2];
    for (int k = 0;; ++k) {
        // The thread index is made opaque once per piece, so that the compiler
        // computes the lane-dependent addresses (the swizzled LDS operand
        // offsets, the state elements' offsets) in each piece instead of once
        // before this loop, where they would stay in registers through every
        // piece's warm-up and set-up as well and spill.
        const int tid = opaque((int)threadIdx.x), lane = tid & 63;
        const int qh = w >> 2, cq = w & 3, r32 = lane & 31, hf = lane >> 5;
        auto sbase = [&]() { return (64 * qh + 4 * hf) * D + 32 * cq + r32; };
        auto sidx = [&](int base, int db, int v) { return base + (32 * db + 8 * (v >> 2) + (v & 3)) * D; };
        __syncthreads();  // the previous piece is done with the tiles, S^T and pc
        if (tid == 0)
            pc = next_piece<OutT>(*reinterpret_cast<const PrefillArgs *>(args_lds),
                                  *reinterpret_cast<const Segmented *>(sp_lds), ws_lds, mode, k, ps, heads_pre,
                                  heads_warm, cpre, bulk, qlist, by_rank);
        __syncthreads();
        const int uh = __builtin_amdgcn_readfirstlane(pc.uh);
        if (uh < 0) break;
        const int ts = __builtin_amdgcn_readfirstlane(pc.ts);
        const float s2 = uniformf(pc.s2);
        const float *s_in = uniform_ptr(pc.s_in);
        const bool s_in_t = __builtin_amdgcn_readfirstlane(pc.s_in_t) != 0;
        // carried-in state
        if (s_in && s_in_t) {
            // S_0 given transposed: element (r, c) at c * D + r
            const int tb = (32 * cq + r32) * D + 64 * qh + 4 * hf;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) S[db][v] = s_in[tb + 32 * db + 8 * (v >> 2) + (v & 3)];
        } else if (s_in) {
            const int sb = sbase();
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) S[db][v] = s_in[sidx(sb, db, v)];
        } else {
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) S[db][v] = 0.f;
        }
        const int comb_g = __builtin_amdgcn_readfirstlane(pc.comb_g);
        if (comb_g > 0)
            combine_start(S, *reinterpret_cast<const Segmented *>(sp_lds), uniform_ptr(pc.u), comb_g,
                          __builtin_amdgcn_readfirstlane(pc.kg), uniform64(pc.covered), s2, qh, cq, lane);

        // this piece's rows: a warm-up over [t0w, t0) (whole sub-blocks, an
        // even number), then its tokens
        const long long warm = uniform64(pc.warm);
        const uint16_t *kw = uniform_ptr(pc.k), *vw = uniform_ptr(pc.v);
        const long long len = uniform64(pc.len);
        const uint16_t *qg = uniform_ptr(pc.q);
        const uint16_t *kg = kw + warm * ts, *vg = vw + warm * ts;
        OutT *og = static_cast<OutT *>(uniform_ptr(pc.o));
        // epilogue: gate rows of this piece and the head's normalisation
        // weights, kept in LDS (read after the first barrier B)
        const uint16_t *gg = NG ? uniform_ptr(pc.gate) : nullptr;
        const float eps = NG ? uniformf(pc.eps) : 0.f;
        if (NG && tid < D / 4)
            *reinterpret_cast<float4 *>(Wn + 4 * tid) = *reinterpret_cast<const float4 *>(uniform_ptr(pc.nw) + 4 * tid);

        // Two register stages: sub-block c is staged in st[c % 2] and its loads
        // are issued two sub-blocks ahead, so about 96 KiB of loads are in flight
        // per CU.
        Stage<true> st0, st1;
        const long long nfull = len / C;
        const int tail = (int)(len - nfull * C);
        const long long nchunks = nfull + (tail > 0);
        auto chunk_len = [&](long long c) { return c < nfull ? C : tail; };
        auto prefetch = [&](Stage<true> &st, long long c) {
            // Past the end the same loads read one row of the last sub-block again
            // (row stride 0; ignored): the count of loads stays fixed, so the
            // compiler's waits stay exact, and almost nothing leaves HBM (a
            // re-read of whole sub-blocks cost about 3% of the call's traffic).
            const bool in = c < nchunks;
            const long long cn = in ? c : nchunks - 1;
            const long long off = cn * C * (long long)ts;
            st.load(qg + off, kg + off, vg + off, in ? ts : 0, in ? chunk_len(cn) : C, tid);
        };
        if (warm > 0) {  // state-only steps, with their own two stages
            // even: pieces start at multiples of 128 tokens and warm_len is one
            const long long nw = warm / C;
            const float bdw = fast_exp2(-s2 * (float)C);
            Stage<false> w0, w1;
            auto wpre = [&](Stage<false> &st, long long c) {
                const long long off = c * C * (long long)ts;
                st.load(nullptr, kw + off, vw + off, ts, C, tid);
            };
            auto wstep = [&](Stage<false> &st, auto &&issue) {
                __builtin_amdgcn_sched_barrier(0);
                __syncthreads();
                st.template store<true>(nullptr, Ks, nullptr, Vds, C, s2, tid);
                issue();
                __syncthreads();
                state_update(S, Ks, Vds, bdw, qh, cq, lane);
            };
            wpre(w0, 0);
            wpre(w1, 1);
            long long c = 0;
            for (; c + 2 < nw; c += 2) {
                wstep(w0, [&] { wpre(w0, c + 2); });
                wstep(w1, [&] { wpre(w1, c + 3); });
            }
            // the last two warm-up steps issue the first two token sub-blocks'
            // loads (the same two loads, in the same order, as without a warm-up)
            wstep(w0, [&] { prefetch(st0, 0); });
            wstep(w1, [&] { prefetch(st1, 1); });
            __syncthreads();  // the last warm-up reads of Ks, Vds are done
        } else if (nchunks > 0) {
            prefetch(st0, 0);
            prefetch(st1, 1);
        }
        write_state_t(Sts[0], S, qh, cq, lane);

        // loop-invariant decay factors
        const int qpos = 32 * qh + r32;                       // query row of this lane's outputs
        const float dq = fast_exp2(-s2 * (float)(qpos + 1));  // d_q for that row
        const bool scorer = w < 3;                            // waves 0..2 own one score block each
        const int qb = w == 0 ? 0 : 1, kb = w == 2 ? 1 : 0;   // (query block, key block)
        float dscore[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int diff = (32 * qb + r32) - (32 * kb + 8 * (v >> 2) + 4 * hf + (v & 3));
            dscore[v] = masked_decay(diff, s2);
        }

        int cur = 0;
        // Per sub-block: (B) tiles visible -> scores, inter-block product, state
        // update -> (C) P visible -> intra-block product, output block to LDS ->
        // (D) output tile visible and every read of this sub-block's tiles done
        // -> full-row output stores. Barrier D of one sub-block also guards the
        // tile writes of the next. The output tile reuses the S^T buffer that
        // the inter-block product just finished reading (it is rewritten only
        // after the next barrier B).
        auto step = [&](long long c, int m, auto full, Stage<true> &st) {
            constexpr bool FULL = decltype(full)::value;
            // gate rows of this sub-block, consumed by the epilogue at its end.
            // They are issued ahead of the prefetch two sub-blocks out: loads
            // complete in order, so the epilogue's wait for them then leaves
            // that prefetch in flight (issued after it, the wait drained it:
            // 0.63 -> 0.61 ms per norm-gate call on the M1 layer)
            uint2 gr[4];
            if constexpr (NG) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = (tid >> 5) + 16 * j;
                    const int rr = FULL || row < m ? row : m - 1;
                    gr[j] = stream_load8(gg + (c * C + rr) * (long long)ts + 4 * (tid & 31));
                }
            }
            st.template store<FULL>(Qs, Ks, Vs, Vds, m, s2, tid);
            if (FULL) prefetch(st, c + 2);
            __syncthreads();  // (B) tiles and S^T of the previous sub-block are visible
            if (scorer) {
                // scores^T block: keys 32kb.., queries 32qb.. ; masked, decayed, to LDS as P
                f32x16 sc;
#pragma unroll
                for (int v = 0; v < 16; ++v) sc[v] = 0.f;
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks)
                    sc = mma(ld_op<L128>(Ks, 32 * kb, 16 * ks, lane), ld_op<L128>(Qs, 32 * qb, 16 * ks, lane), sc);
#pragma unroll
                for (int gv = 0; gv < 4; ++gv) {
                    bf16x4 p;
#pragma unroll
                    for (int r = 0; r < 4; ++r) p[r] = static_cast<__bf16>(mask_mul(sc[4 * gv + r], dscore[4 * gv + r]));
                    *reinterpret_cast<bf16x4 *>(Ps + LP::off(32 * qb + r32, 32 * kb + 8 * gv + 4 * hf)) = p;
                }
            }

            // inter-block part: O^T = S^T (Q ⊙ d_q)^T
            f32x16 o;
#pragma unroll
            for (int v = 0; v < 16; ++v) o[v] = 0.f;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                o = mma(ld_op<L128>(Sts[cur], 32 * cq, 16 * ks, lane), ld_op<L128>(Qs, 32 * qh, 16 * ks, lane), o);
            o *= dq;

            // state: S = e^{-s m} S + K^T (V ⊙ d_k), then S^T (bf16) for the next sub-block
            state_update(S, Ks, Vds, fast_exp2(-s2 * (float)m), qh, cq, lane);
            write_state_t(Sts[cur ^ 1], S, qh, cq, lane);
            __syncthreads();  // (C) P is visible

            // intra-block part: O^T += V^T P^T over the causal key range
#pragma unroll
            for (int ks = 0; ks < C / 16; ++ks) {
                if (ks >= 2 * (qh + 1)) break;
                o = mma(ld_op_t<L128>(Vs, 32 * cq, 16 * ks, lane), ld_op<LP>(Ps, 32 * qh, 16 * ks, lane), o);
            }
            float *Os = reinterpret_cast<float *>(Sts[cur]);
            stage_out(Os, o, qh, cq, lane);
            if constexpr (NG) row_sumsq(Rss, o, qh, cq, lane);
            __syncthreads();  // (D)
            if constexpr (NG)
                store_rows_norm_gate<FULL>(og + c * C * (long long)ts, ts, Os, Rss, m, tid, gr,
                                           *reinterpret_cast<const float4 *>(Wn + 4 * (tid & 31)), eps);
            else
                store_rows<FULL>(og + c * C * (long long)ts, ts, Os, m, tid);
            cur ^= 1;
        };
        long long c = 0;
        for (; c + 1 < nfull; c += 2) {
            step(c, C, std::true_type{}, st0);
            step(c + 1, C, std::true_type{}, st1);
        }
        if (c < nfull) step(c, C, std::true_type{}, st0);
        if (tail > 0) {  // sub-block nfull is staged in st[nfull % 2]
            if (nfull & 1)
                step(nfull, tail, std::false_type{}, st1);
            else
                step(nfull, tail, std::false_type{}, st0);
        }

        // the end state (pc is unchanged until the next piece)
        const int end = __builtin_amdgcn_readfirstlane(pc.end);
        if (end == 1) {  // the final state
            float *dst = uniform_ptr(pc.dst);
            const int sb = sbase();
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) dst[sidx(sb, db, v)] = S[db][v];
        } else if (end == 2) {  // a warm piece ending inside its pair: record a NaN or Inf
            bool bad = false;
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) bad |= nonfinite(S[db][v]);
            if (bad) {  // rare: every entry of this thread's state blocks is in column 32 cq + r32
                int *rec = pc.rec;
                const int sb = sbase();
#pragma unroll
                for (int db = 0; db < 2; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (nonfinite(S[db][v])) {
                            const int e = sidx(sb, db, v);
                            atomicOr(reinterpret_cast<unsigned *>(rec + kRecEntBad) + (e >> 5), 1u << (e & 31));
                        }
                atomicMin(rec + kRecColCut + 32 * cq + r32, pc.cut);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Value-slice variant, for launches with too few (sequence, head) pairs to fill
// the GPU with whole heads (batch-1 prefill: 64 pairs for 256 CUs). Output
// columns J depend only on V[:, J] and S[:, J], so a head's 128 value columns
// split into 4 independent 32-column workgroups with no pre-pass and no extra
// HBM traffic: the four workgroups of a head read the same q and k tiles, and
// the launch places them on one XCD so the repeats hit that XCD's L2.
// Per 64-token sub-block the 8 waves split: waves 0..2 one causal 32x32 score
// block each; waves 3, 4 the two 32x32 output blocks (inter then intra part);
// waves 5, 6, 7 and 0 one 32x32 state block each (keys 32*db.., 32 columns).
constexpr int NSL = 4;          // value slices per head
constexpr int SW = D / NSL;     // 32 value columns per workgroup
constexpr int VP = SW + 8;      // LDS pitch (elements) of the V slice tiles
constexpr int OSS = SW + 4;     // fp32 pitch of the staged output slice

// Register staging for a slice workgroup: q, k as in Stage (tokens (t/16) + 32i,
// elements 8(t%16)..), v slice 8 bytes per thread (token t/8, columns 4(t%8)..).
struct SliceStage {
    uint4 q[2], k[2];
    uint2 v;

    __device__ void load(const uint16_t *qg, const uint16_t *kg, const uint16_t *vg, int ts, int m,
                         int tid) {
        const int seg = tid & 15;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = (tid >> 4) + 32 * i;
            const int row = (t < m ? t : m - 1) * ts + 8 * seg;
            // q and k rows are read by all four slice workgroups of the head
            // (on one XCD): default cache policy, so the repeats hit L2
            // (10% faster than non-temporal loads on 1 x 3000 x 64 heads)
            q[i] = *reinterpret_cast<const uint4 *>(qg + row);
            k[i] = *reinterpret_cast<const uint4 *>(kg + row);
        }
        const int vt = tid >> 3;
        v = stream_load8(vg + (vt < m ? vt : m - 1) * ts + 4 * (tid & 7));
    }

    __device__ void store(__bf16 *Qs, __bf16 *Ks, __bf16 *Vs, __bf16 *Vds, int m, float s2, int tid) {
        const int seg = tid & 15;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = (tid >> 4) + 32 * i;
            const bool in = t < m;
            *reinterpret_cast<uint4 *>(Qs + L128::off(t, 8 * seg)) = keep_if(in, q[i]);
            *reinterpret_cast<uint4 *>(Ks + L128::off(t, 8 * seg)) = keep_if(in, k[i]);
        }
        const int vt = tid >> 3;
        const bool in = vt < m;
        const uint2 vv = make_uint2(in ? v.x : 0u, in ? v.y : 0u);
        *reinterpret_cast<uint2 *>(Vs + vt * VP + 4 * (tid & 7)) = vv;
        const float dk = in ? fast_exp2(-s2 * (float)(m - 1 - vt)) : 0.f;
        const uint4 sc = scale_bf16x8(make_uint4(vv.x, vv.y, 0u, 0u), dk);
        *reinterpret_cast<uint2 *>(Vds + vt * VP + 4 * (tid & 7)) = make_uint2(sc.x, sc.y);
    }
};

template <bool FULL>
__device__ __forceinline__ void store_slice_rows(float *out, long long ts, const float *Os, int m,
                                                 int tid) {
    const int row = tid >> 3, col = 4 * (tid & 7);
    const float4 x = *reinterpret_cast<const float4 *>(Os + row * OSS + col);
    if (FULL || row < m) stream_store(out + row * ts + col, x);
}
template <bool FULL>
__device__ __forceinline__ void store_slice_rows(__bf16 *out, long long ts, const float *Os, int m,
                                                 int tid) {
    const int row = tid >> 3, col = 4 * (tid & 7);
    const float4 x = *reinterpret_cast<const float4 *>(Os + row * OSS + col);
    const bf16x4 y = {static_cast<__bf16>(x.x), static_cast<__bf16>(x.y), static_cast<__bf16>(x.z),
                      static_cast<__bf16>(x.w)};
    if (FULL || row < m) stream_store_bits(out + row * ts + col, y);
}

template <typename OutT>
__global__ __launch_bounds__(NT) void slice_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 Qs[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Ks[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Vs[C * VP];
    __shared__ __attribute__((aligned(16))) __bf16 Vds[C * VP];
    __shared__ __attribute__((aligned(16))) __bf16 Sts[2][SW * D];
    __shared__ __attribute__((aligned(16))) __bf16 Ps[C * PW];
    __shared__ __attribute__((aligned(16))) float Os[C * OSS];

    // XCD-aware mapping: workgroups are dealt round-robin over the 8 XCDs, so
    // v = (bid % 8) * (nwg / 8) + bid / 8 gives each XCD a contiguous run of v,
    // and the 4 slices of a head share one XCD.
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int vid = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
    const int slice = vid % NSL, uh = vid / NSL;
    const int h = uh % a.heads, n = uh / a.heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31, hf = lane >> 5;

    const SeqRange sr = sequence_of(a, n);
    const long long len = sr.len;
    const int ts = a.heads * D;
    const long long base = (sr.start * a.heads + h) * (long long)D;
    const uint16_t *qg = static_cast<const uint16_t *>(a.q) + base;
    const uint16_t *kg = static_cast<const uint16_t *>(a.k) + base;
    const uint16_t *vg = static_cast<const uint16_t *>(a.v) + base + slice * SW;
    OutT *og = static_cast<OutT *>(a.o) + base + slice * SW;
    const float s2 = a.slopes[h] * LOG2E;

    // roles
    const bool scorer = w < 3;
    const int qb = w == 0 ? 0 : 1, kb = w == 2 ? 1 : 0;
    const bool outw = (w == 3 || w == 4);
    const int qh = w - 3;                       // output block of waves 3, 4
    const bool stw = (w == 0 || w >= 5);        // state block owners
    const int db = w == 0 ? 3 : w - 5;          // their key block

    // state block S[32db + 8(v/4) + 4hf + v%4][slice*32 + r32]
    f32x16 S;
    const long long sb = (long long)uh * D * D + slice * SW;
    auto sidx = [&](int v) { return (32 * db + 8 * (v >> 2) + 4 * hf + (v & 3)) * D + r32; };
#pragma unroll
    for (int v = 0; v < 16; ++v) S[v] = (stw && a.state_in) ? a.state_in[sb + sidx(v)] : 0.f;
    auto write_st = [&](__bf16 *dst) {
#pragma unroll
        for (int gv = 0; gv < 4; ++gv) {
            bf16x4 x;
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] = static_cast<__bf16>(S[4 * gv + r]);
            *reinterpret_cast<bf16x4 *>(dst + L128::off(r32, 32 * db + 8 * gv + 4 * hf)) = x;
        }
    };
    if (stw) write_st(Sts[0]);

    const int qpos = 32 * qh + r32;
    const float dq = fast_exp2(-s2 * (float)(qpos + 1));
    float dscore[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int diff = (32 * qb + r32) - (32 * kb + 8 * (v >> 2) + 4 * hf + (v & 3));
        dscore[v] = masked_decay(diff, s2);
    }

    SliceStage st0, st1;
    const long long nfull = len / C;
    const int tail = (int)(len - nfull * C);
    const long long nchunks = nfull + (tail > 0);
    auto chunk_len = [&](long long c) { return c < nfull ? C : tail; };
    auto prefetch = [&](SliceStage &st, long long c) {
        // past the end one row is read again (row stride 0; ignored)
        const bool in = c < nchunks;
        const long long cn = in ? c : nchunks - 1;
        const long long off = cn * C * (long long)ts;
        st.load(qg + off, kg + off, vg + off, in ? ts : 0, in ? chunk_len(cn) : C, tid);
    };
    if (nchunks > 0) {
        prefetch(st0, 0);
        prefetch(st1, 1);
    }

    int cur = 0;
    auto step = [&](long long c, int m, auto full, SliceStage &st) {
        constexpr bool FULL = decltype(full)::value;
        st.store(Qs, Ks, Vs, Vds, m, s2, tid);
        if (FULL) prefetch(st, c + 2);
        __syncthreads();  // (B) tiles and S^T of the previous sub-block are visible

        f32x16 o;
        if (scorer) {
            f32x16 sc;
#pragma unroll
            for (int v = 0; v < 16; ++v) sc[v] = 0.f;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                sc = mma(ld_op<L128>(Ks, 32 * kb, 16 * ks, lane), ld_op<L128>(Qs, 32 * qb, 16 * ks, lane), sc);
#pragma unroll
            for (int gv = 0; gv < 4; ++gv) {
                bf16x4 p;
#pragma unroll
                for (int r = 0; r < 4; ++r) p[r] = static_cast<__bf16>(mask_mul(sc[4 * gv + r], dscore[4 * gv + r]));
                *reinterpret_cast<bf16x4 *>(Ps + LP::off(32 * qb + r32, 32 * kb + 8 * gv + 4 * hf)) = p;
            }
        }
        if (outw) {  // inter-block part O^T = S^T (Q ⊙ d_q)^T
#pragma unroll
            for (int v = 0; v < 16; ++v) o[v] = 0.f;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                o = mma(ld_op<L128>(Sts[cur], 0, 16 * ks, lane), ld_op<L128>(Qs, 32 * qh, 16 * ks, lane), o);
            o *= dq;
        }
        if (stw) {  // S = e^{-s m} S + K^T (V ⊙ d_k) for keys 32db..
            S *= fast_exp2(-s2 * (float)m);
#pragma unroll
            for (int ks = 0; ks < C / 16; ++ks)
                S = mma(ld_op_t<L128>(Ks, 32 * db, 16 * ks, lane), ld_op_t<LPad<VP>>(Vds, 0, 16 * ks, lane), S);
            write_st(Sts[cur ^ 1]);
        }
        __syncthreads();  // (C) P and the new S^T are visible

        if (outw) {  // intra-block part O^T += V^T P^T, then stage the block
#pragma unroll
            for (int ks = 0; ks < C / 16; ++ks) {
                if (ks >= 2 * (qh + 1)) break;
                o = mma(ld_op_t<LPad<VP>>(Vs, 0, 16 * ks, lane), ld_op<LP>(Ps, 32 * qh, 16 * ks, lane), o);
            }
#pragma unroll
            for (int gv = 0; gv < 4; ++gv)
                *reinterpret_cast<float4 *>(Os + (32 * qh + r32) * OSS + 8 * gv + 4 * hf) =
                    make_float4(o[4 * gv], o[4 * gv + 1], o[4 * gv + 2], o[4 * gv + 3]);
        }
        __syncthreads();  // (D) output slice staged; every tile read of this sub-block done
        store_slice_rows<FULL>(og + c * C * (long long)ts, ts, Os, m, tid);
        cur ^= 1;
    };
    long long c = 0;
    for (; c + 1 < nfull; c += 2) {
        step(c, C, std::true_type{}, st0);
        step(c + 1, C, std::true_type{}, st1);
    }
    if (c < nfull) step(c, C, std::true_type{}, st0);
    if (tail > 0) {
        if (nfull & 1)
            step(nfull, tail, std::false_type{}, st1);
        else
            step(nfull, tail, std::false_type{}, st0);
    }

    if (a.state_out && stw) {
#pragma unroll
        for (int v = 0; v < 16; ++v) a.state_out[sb + sidx(v)] = S[v];
    }
}

// ---------------------------------------------------------------------------
// Finishing pass of the warm-up route: one workgroup per (unit, head) pair;
// pairs on the pre-pass route exit at once. A piece that starts inside its pair
// builds its carried-in state from a window of earlier tokens, so it cannot see
// a NaN or Inf from before that window, which the exact operator carries
// forward: it stays in the state entries it reached, and every later output in
// the value columns of those entries is non-finite. The pieces that ended
// inside the pair recorded where their end states held one (warm_records);
// this pass puts NaN in every output of column c from the earliest such end in
// that column on (in whole rows with the norm-gate epilogue, whose
// normalisation spreads it over the row) and in each final-state entry that
// was non-finite at some such end. It also writes the final state of empty
// sequences (S_0, or zero) and, for in-place calls (state_out == state_in),
// copies the final state that the main pass left in the workspace: writing it
// there directly could race with the reads of S_0 by the pair's other pieces.

template <typename OutT, bool NG>
__global__ __launch_bounds__(NT) void finish_kernel(PrefillArgs a, Segmented sp, float *ws) {
    __shared__ int colcut[D];
    __shared__ int mincut;
    const int tid = threadIdx.x;
    const int uh = blockIdx.x, h = uh % a.heads, n = uh / a.heads;
    const long long len = SeqLens{a.cu_seqlens, a.total_tokens, a.seqlen}.len(n);
    const size_t sb = (size_t)uh * D * D;
    const bool in_place = a.state_in && a.state_in == a.state_out;
    if (takes_prepass(sp, a.slopes[h] * LOG2E)) {  // the pre-pass route: only an in-place final state
        if (in_place) {
            const float4 *src = reinterpret_cast<const float4 *>(sp.final_state(sp.unit(ws, uh)));
            float4 *dst = reinterpret_cast<float4 *>(a.state_out + sb);
#pragma unroll
            for (int j = 0; j < kStateF4; ++j) dst[threadIdx.x + NT * j] = src[threadIdx.x + NT * j];
        }
        return;
    }
    if (len == 0) {  // no piece covers the pair: the final state is S_0
        if (a.state_out && a.state_out != a.state_in)
            for (int i = tid; i < D * D; i += NT) {
                float x = 0.f;
                if (a.state_in) x = a.state_in_t ? a.state_in[sb + (i % D) * D + i / D] : a.state_in[sb + i];
                a.state_out[sb + i] = x;
            }
        return;
    }
    const int *rec = warm_records(sp, ws, uh);
    if (tid == 0) mincut = kNoCut;
    __syncthreads();
    if (tid < D) {
        colcut[tid] = rec[kRecColCut + tid];
        atomicMin(&mincut, colcut[tid]);
    }
    __syncthreads();
    const int first = mincut;
    if (first != kNoCut) {
        // rows t >= colcut[c] in column c; 32 threads per row (4 columns each),
        // NT / 32 rows at a time
        const int col = 4 * (tid & 31);
        const long long base = sequence_of(a, n).start;
        OutT *o = static_cast<OutT *>(a.o);
        int cut4[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) cut4[x] = NG ? first : colcut[col + x];
        for (long long t = first + (tid >> 5); t < len; t += NT / 32) {
            OutT *row = o + ((base + t) * a.heads + h) * (long long)D + col;
#pragma unroll
            for (int x = 0; x < 4; ++x)
                if (t >= cut4[x]) poison(row + x);
        }
    }
    if (a.state_out && (in_place || first != kNoCut)) {
        // this thread's state elements: float4 tid + NT j (j < kStateF4)
        const unsigned *bad = reinterpret_cast<const unsigned *>(rec + kRecEntBad);
        const float4 *src = reinterpret_cast<const float4 *>(in_place ? sp.final_state(sp.unit(ws, uh))
                                                                      : a.state_out + sb);
        float4 *dst = reinterpret_cast<float4 *>(a.state_out + sb);
#pragma unroll
        for (int j = 0; j < kStateF4; ++j) {
            const int f = tid + NT * j;
            float4 x = src[f];
            const unsigned b = first != kNoCut ? (bad[f >> 3] >> (4 * (f & 7))) & 0xfu : 0u;  // entries 4f .. 4f+3
            if (b & 1) x.x = __builtin_nanf("");
            if (b & 2) x.y = __builtin_nanf("");
            if (b & 4) x.z = __builtin_nanf("");
            if (b & 8) x.w = __builtin_nanf("");
            dst[f] = x;
        }
    }
}

template <typename OutT>
hipError_t launch(const PrefillArgs &a, const PrefillPlan &p, void *workspace, hipStream_t stream) {
    clear_pending_error();
    const long long uh = (long long)a.units * a.heads;
    // a value-slice workgroup sees 32 of a row's 128 columns: no row epilogue
    if (p.value_slices == NSL && (a.ng.gate || a.state_in_t)) return hipErrorInvalidValue;
    if (p.value_slices == NSL) {
        hipLaunchKernelGGL((slice_kernel<OutT>), dim3((unsigned)(uh * NSL)), dim3(NT), 0, stream, a);
        return hipGetLastError();
    }
    float *ws = static_cast<float *>(workspace);
    const Segmented sp{p.segments, p.pieces, p.seg_len, p.piece_len};
    if (p.segments > 1) {
        // the kernels' per-plan tables hold every pair and workgroup of a segmented plan
        if (uh >= kMaxPairs) return hipErrorInvalidValue;
        // working pre-pass workgroups: at most kPrepassActive + uh (see piece_state_kernel)
        const long long pre = uh * p.pieces < kPrepassActive + uh ? uh * p.pieces : kPrepassActive + uh;
        hipLaunchKernelGGL(piece_state_kernel, dim3((unsigned)pre), dim3(NT), 0, stream, a, sp, ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)(uh * p.segments));
    if (a.ng.gate)
        hipLaunchKernelGGL((head_kernel<OutT, true>), grid, dim3(NT), 0, stream, a, sp, ws);
    else
        hipLaunchKernelGGL((head_kernel<OutT, false>), grid, dim3(NT), 0, stream, a, sp, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.segments == 1) return e;
    if (a.ng.gate)
        hipLaunchKernelGGL((finish_kernel<OutT, true>), dim3((unsigned)uh), dim3(NT), 0, stream, a, sp, ws);
    else
        hipLaunchKernelGGL((finish_kernel<OutT, false>), dim3((unsigned)uh), dim3(NT), 0, stream, a, sp, ws);
    return hipGetLastError();
}

}  // namespace

hipError_t load_prefill_heads_code() {
    hipFuncAttributes attr;
    return hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(&head_kernel<float, false>));
}

hipError_t launch_prefill_heads(const PrefillArgs &a, const PrefillPlan &plan, void *workspace,
                                lt_dtype out_dtype, hipStream_t stream) {
    return out_dtype == LT_F32 ? launch<float>(a, plan, workspace, stream)
                               : launch<__bf16>(a, plan, workspace, stream);
}

}  // namespace lt
