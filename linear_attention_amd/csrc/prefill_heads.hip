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
//  * Heads whose decay ends their memory within a segment skip the pre-pass:
//    their segments start from a zero state, and a correction pass adds the
//    missed carried-in term e^{-s(t+1)} q_t S_in to each segment's first
//    tokens (with the norm-gate epilogue the main kernel leaves those rows raw
//    in y and the correction pass also normalises and gates them).
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

// raw: store o itself (every factor replaced by 1, by a select).
template <bool FULL, typename OutT>
__device__ __forceinline__ void store_rows_norm_gate(OutT *out, long long ts, const float *Os,
                                                     const float *rss, int m, int tid,
                                                     const uint2 (&gr)[4], float4 w, float eps, bool raw) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = (tid >> 5) + 16 * j, col = 4 * (tid & 31);
        const float4 x = *reinterpret_cast<const float4 *>(Os + ooff(row, col));
        const float4 p = *reinterpret_cast<const float4 *>(rss + 4 * row);
        const float inv = __builtin_amdgcn_rsqf((p.x + p.y + p.z + p.w) * (1.f / D) + eps);
        const float g0 = __uint_as_float(gr[j].x << 16), g1 = __uint_as_float(gr[j].x & 0xffff0000u);
        const float g2 = __uint_as_float(gr[j].y << 16), g3 = __uint_as_float(gr[j].y & 0xffff0000u);
        const float f0 = raw ? 1.f : inv * w.x * sigmoid(g0), f1 = raw ? 1.f : inv * w.y * sigmoid(g1);
        const float f2 = raw ? 1.f : inv * w.z * sigmoid(g2), f3 = raw ? 1.f : inv * w.w * sigmoid(g3);
        const float4 y = make_float4(x.x * f0, x.y * f1, x.z * f2, x.w * f3);
        if (FULL || row < m) put4(out + row * ts + col, y);
    }
}

// Pre-pass: workgroup (unit, head, piece j) runs the state update over the
// full 64-token sub-blocks of its group of pieces without outputs, writing its
// state and, if a segment boundary falls strictly inside the group, B_g on the
// way.
__global__ __launch_bounds__(NT, 4) void piece_state_kernel(PrefillArgs a, Segmented sp, float *ws) {
    __shared__ __attribute__((aligned(16))) __bf16 Ks[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Vds[C * D];

    // workgroup b takes group b % gph of (unit, head) b / gph, gph groups of
    // kgr pieces per head; the working workgroups are the first U * gph, which
    // the hardware spreads over all XCDs. The group's state goes to the slot
    // of its last piece.
    const int kgr = prepass_group(a.slopes, a.heads, a.units, sp);
    const int gph = (sp.pieces + kgr - 1) / kgr;
    if ((int)blockIdx.x >= a.units * a.heads * gph) return;
    const int j = (blockIdx.x % gph) * kgr;
    const int uh = blockIdx.x / gph;
    const int h = uh % a.heads, n = uh / a.heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qh = w >> 2, cq = w & 3, r32 = lane & 31, hf = lane >> 5;

    const float s2 = a.slopes[h] * LOG2E;
    if (fix_head(s2, sp.seg_len, sp.fix_osz)) return;  // local-start segments: no pre-pass
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
        const long long off = (c < nch ? c : nch - 1) * C * (long long)ts;
        st.load(nullptr, kg + off, vg + off, ts, C, tid);
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

template <typename OutT, bool NG>
__global__ __launch_bounds__(NT) void head_kernel(PrefillArgs a, Segmented sp, float *ws) {
    __shared__ __attribute__((aligned(16))) __bf16 Qs[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Ks[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Vs[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Vds[C * D];
    __shared__ __attribute__((aligned(16))) __bf16 Sts[2][D * D];
    __shared__ __attribute__((aligned(16))) __bf16 Ps[C * PW];

    const int segments = sp.segments;
    const long long seg_len = sp.seg_len;
    const int g = blockIdx.x % segments;
    const int slot = blockIdx.x / segments;
    const int h = slot % a.heads;
    const int tid = threadIdx.x, lane = tid & 63;
    // Packed batches of up to kRankUnits sequences run their longest sequences
    // first: unit slot r takes the sequence of rank r by length (descending,
    // ties by index), so the long whole-sequence workgroups do not start last
    // and leave the end of the launch to a few CUs.
    int n = slot / a.heads;
    if (a.cu_seqlens && a.units <= kRankUnits) {
        __shared__ long long lens[kRankUnits];
        __shared__ int by_rank[kRankUnits];
        if (tid < a.units) lens[tid] = sequence_of(a, tid).len;
        __syncthreads();
        if (tid < a.units) {
            const long long li = lens[tid];
            int r = 0;
            for (int j = 0; j < a.units; ++j) r += lens[j] > li || (lens[j] == li && j < tid);
            by_rank[r] = tid;
        }
        __syncthreads();
        n = by_rank[n];
    }
    const int uh = n * a.heads + h;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qh = w >> 2, cq = w & 3, r32 = lane & 31, hf = lane >> 5;

    const SeqRange sr = sequence_of(a, n);
    const int gused = sp.used(sr.len);  // segments this sequence has
    if (g >= gused) return;
    const long long seg0 = (long long)g * seg_len;
    long long len = sr.len - seg0;
    len = len < 0 ? 0 : (len > seg_len ? seg_len : len);
    const int ts = a.heads * D;
    const long long base = ((sr.start + seg0) * a.heads + h) * (long long)D;
    const uint16_t *qg = static_cast<const uint16_t *>(a.q) + base;
    const uint16_t *kg = static_cast<const uint16_t *>(a.k) + base;
    const uint16_t *vg = static_cast<const uint16_t *>(a.v) + base;
    OutT *og = static_cast<OutT *>(a.o) + base;
    const float s2 = a.slopes[h] * LOG2E;
    // epilogue: gate rows of this (sequence, head) and the head's normalisation
    // weights, kept in LDS (read after the first barrier B)
    __shared__ __attribute__((aligned(16))) float Wn[NG ? D : 1];
    __shared__ __attribute__((aligned(16))) float Rss[NG ? C * 4 : 1];  // per-row partial sums of o^2
    const uint16_t *gg = NG ? static_cast<const uint16_t *>(a.ng.gate) + base : nullptr;
    if (NG && tid < D / 4)
        *reinterpret_cast<float4 *>(Wn + 4 * tid) = *reinterpret_cast<const float4 *>(a.ng.norm_weight + h * D + 4 * tid);

    // ---- carried-in state of this segment (the combine pass wrote it for
    // segmented plans; on local-start segments segment 0 reads S_0 itself and
    // the final state is written by a later kernel; either way an in-place
    // state update never races with this read)
    f32x16 S[2];
    auto sidx = [&](int db, int v) {
        return (64 * qh + 32 * db + 8 * (v >> 2) + 4 * hf + (v & 3)) * D + 32 * cq + r32;
    };
    // local-start segments: segment 0 starts from S_0, the others from zero
    // (the correction pass adds their carried-in term afterwards)
    const bool fix = segments > 1 && fix_head(s2, seg_len, sp.fix_osz);
    const float *s_in = segments > 1 && !fix
                            ? sp.start_state(sp.unit(ws, uh), g)
                            : ((segments == 1 || g == 0) && a.state_in ? a.state_in + (size_t)uh * D * D : nullptr);
    if (s_in && (segments == 1 || fix) && a.state_in_t) {
        // S_0 given transposed: element (r, c) at c * D + r
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 64 * qh + 32 * db + 8 * (v >> 2) + 4 * hf + (v & 3), c = 32 * cq + r32;
                S[db][v] = s_in[c * D + r];
            }
    } else if (s_in) {
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) S[db][v] = s_in[sidx(db, v)];
    } else {
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) S[db][v] = 0.f;
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

    // Two register stages: sub-block c is staged in st[c % 2] and its loads are
    // issued two sub-blocks ahead, so about 96 KiB of loads are in flight per CU.
    Stage<true> st0, st1;
    const long long nfull = len / C;
    const int tail = (int)(len - nfull * C);
    const long long nchunks = nfull + (tail > 0);
    auto chunk_len = [&](long long c) { return c < nfull ? C : tail; };
    auto prefetch = [&](Stage<true> &st, long long c) {
        // past the end, re-read the last sub-block (ignored) to keep the count fixed
        const long long cn = c < nchunks ? c : nchunks - 1;
        const long long off = cn * C * (long long)ts;
        st.load(qg + off, kg + off, vg + off, ts, chunk_len(cn), tid);
    };
    if (nchunks > 0) {
        prefetch(st0, 0);
        prefetch(st1, 1);
    }

    int cur = 0;
    // Per sub-block: (B) tiles visible -> scores, inter-block product, state
    // update -> (C) P visible -> intra-block product, output block to LDS ->
    // (D) output tile visible and every read of this sub-block's tiles done ->
    // full-row output stores. Barrier D of one sub-block also guards the tile
    // writes of the next. The output tile reuses the S^T buffer that the
    // inter-block product just finished reading (it is rewritten only after the
    // next barrier B).
    // norm-gate on a local-start segment g >= 1: the sub-blocks of its first
    // raw_rows rows store the raw output to y (the epilogue's scale replaced
    // by 1, a select rather than a second store path), which the correction
    // pass finishes
    const long long raw_rows = NG && fix && g > 0 ? ng_fix_rows(s2, seg_len, len) : 0;
    auto step = [&](long long c, int m, auto full, Stage<true> &st) {
        constexpr bool FULL = decltype(full)::value;
        // gate rows of this sub-block, consumed by the epilogue at its end. They
        // are issued ahead of the prefetch two sub-blocks out: loads complete in
        // order, so the epilogue's wait for them then leaves that prefetch in
        // flight (issued after it, the wait drained it: 0.63 -> 0.61 ms per
        // norm-gate call on the M1 layer)
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
                                       *reinterpret_cast<const float4 *>(Wn + 4 * (tid & 31)), a.ng.eps,
                                       c * C < raw_rows);
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

    if (fix) {  // end state of this local-start segment, for the correction pass
        float *u = sp.unit(ws, uh);
        float *dst = sp.start_state(u, g);
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) dst[sidx(db, v)] = S[db][v];
        if (g + 1 < segments) flag_end_state(end_flags(sp, u, g), S, w, lane);
    } else if (a.state_out && g == gused - 1) {
        const long long sb = (long long)uh * D * D;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) a.state_out[sb + sidx(db, v)] = S[db][v];
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
        const long long cn = c < nchunks ? c : nchunks - 1;
        const long long off = cn * C * (long long)ts;
        st.load(qg + off, kg + off, vg + off, ts, chunk_len(cn), tid);
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

// o[t] += e^{-s(t+1)} q[t] S_in(g) for the first fix_len tokens t of segment g
// (g >= 1), in 64-token chunks. The chunks of all (unit, head, segment) pairs
// are numbered in pair order and cut into equal contiguous ranges, one per
// workgroup (the pairs' chunk counts differ with the decay by up to two orders
// of magnitude); consecutive ranges go to workgroups on one XCD, so the few
// workgroups that share a pair read its end states through one L2. A workgroup
// forms S_in(g) from the end states E_0..E_{g-1} the main pass left
// (S_in(1) = E_0, S_in(j+1) = e^{-s len_j} S_in(j) + E_j) and loads the next
// chunk's q and o rows before the current chunk's product, which is the main
// kernel's inter-block one (S^T in bf16 on MFMA, Q from an LDS tile). The first
// `nfinal` workgroups instead write the final state of each local-start head,
// e^{-s len_{G-1}} S_in(G-1) + E_{G-1}, kFinalSlices workgroups per head.
constexpr int kFixWorkgroups = 512;                // two per CU; a multiple of 8 (XCDs)


// The rows of o a thread adds to (loaded before the product, so their latency
// overlaps it): fp32 rows (t/32) + 16j, 4 columns at 4(t%32); bf16 rows
// (t/16) + 32j, 8 columns at 8(t%16). Rows >= m read row m-1 and are not stored.
// Offsets from the chunk's first row fit in 32 bits (64 rows). Sized by the
// output type, so that a copy moves only loaded registers.
template <typename OutT>
struct OutRows;
template <>
struct OutRows<float> {
    uint4 y[4];
    __device__ void load(const float *out, int ts, int m, int tid) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = (tid >> 5) + 16 * j;
            y[j] = *reinterpret_cast<const uint4 *>(out + (unsigned)((row < m ? row : m - 1) * ts + 4 * (tid & 31)));
        }
    }
    __device__ void add_store(float *out, int ts, const float *Os, int m, int tid) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = (tid >> 5) + 16 * j, col = 4 * (tid & 31);
            const float4 x = *reinterpret_cast<const float4 *>(Os + ooff(row, col));
            if (row < m)
                *reinterpret_cast<float4 *>(out + (unsigned)(row * ts + col)) =
                    make_float4(__uint_as_float(y[j].x) + x.x, __uint_as_float(y[j].y) + x.y,
                                __uint_as_float(y[j].z) + x.z, __uint_as_float(y[j].w) + x.w);
        }
    }
};
template <>
struct OutRows<__bf16> {
    uint4 y[2];
    __device__ void load(const __bf16 *out, int ts, int m, int tid) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = (tid >> 4) + 32 * j;
            y[j] = *reinterpret_cast<const uint4 *>(out + (unsigned)((row < m ? row : m - 1) * ts + 8 * (tid & 15)));
        }
    }
    __device__ void add_store(__bf16 *out, int ts, const float *Os, int m, int tid) const {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = (tid >> 4) + 32 * j, col = 8 * (tid & 15);
            const float4 x0 = *reinterpret_cast<const float4 *>(Os + ooff(row, col));
            const float4 x1 = *reinterpret_cast<const float4 *>(Os + ooff(row, col + 4));
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            const uint32_t w[4] = {y[j].x, y[j].y, y[j].z, y[j].w};
            uint32_t r[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const __bf16 lo = static_cast<__bf16>(__uint_as_float(w[i] << 16) + xs[2 * i]);
                const __bf16 hi = static_cast<__bf16>(__uint_as_float(w[i] & 0xffff0000u) + xs[2 * i + 1]);
                uint16_t ulo, uhi;
                __builtin_memcpy(&ulo, &lo, 2);
                __builtin_memcpy(&uhi, &hi, 2);
                r[i] = (uint32_t)ulo | ((uint32_t)uhi << 16);
            }
            if (row < m) *reinterpret_cast<uint4 *>(out + row * ts + col) = make_uint4(r[0], r[1], r[2], r[3]);
        }
    }
};

// One chunk of the correction: rows [t0, t0 + m) of segment g of pair `pair`.
template <typename OutT>
struct FixChunk {
    const uint16_t *q, *gate;
    OutT *o;
    long long t0;
    int m, pair, uh, g, h;
    float s2;
};

// Rows a correction pass treats in segment g of a local-start head (the chunk
// count and the chunk contents must agree on it).
template <bool NG>
__device__ __forceinline__ long long fix_rows(float s2, long long seg_len, long long len) {
    if constexpr (NG) {
        return ng_fix_rows(s2, seg_len, len);
    } else {
        const long long fl = fix_len(s2, seg_len);
        return fl < len ? fl : len;
    }
}

template <typename OutT, bool NG>
__device__ __forceinline__ FixChunk<OutT> fix_chunk(const PrefillArgs &a, const Segmented &sp,
                                                    const long long *first, const long long *prows,
                                                    long long j, int &p) {
    while (first[p + 1] <= j) ++p;
    p = __builtin_amdgcn_readfirstlane(p);  // the same for every lane
    FixChunk<OutT> x;
    const int gs = sp.segments - 1;
    x.pair = p;
    x.uh = p / gs;
    x.g = 1 + p % gs;
    const int h = x.uh % a.heads, n = x.uh / a.heads;
    x.h = h;
    x.s2 = a.slopes[h] * LOG2E;
    const long long T = uniform64(prows[p]);
    x.t0 = uniform64((j - first[p]) * C);
    x.m = (int)(T - x.t0 < C ? T - x.t0 : C);
    const long long row = uniform64(sequence_of(a, n).start) + (long long)x.g * sp.seg_len + x.t0;
    const long long off = (row * a.heads + h) * (long long)D;
    x.q = static_cast<const uint16_t *>(a.q) + off;
    x.gate = NG ? static_cast<const uint16_t *>(a.ng.gate) + off : nullptr;
    x.o = static_cast<OutT *>(a.o) + off;
    return x;
}

// Norm-gate correction rows: the raw output the main pass left in y, and the
// gate, for rows (tid/32) + 16j, columns 4(tid%32)..+3 (the epilogue's layout).
// finish() adds the staged correction, normalises each row (its 32 lanes
// reduce the sum of squares), gates, and stores y.
template <typename OutT>
struct NgRows {
    using Raw = typename std::conditional<sizeof(OutT) == 4, uint4, uint2>::type;
    Raw y[4];
    uint2 gt[4];
    __device__ void load(const OutT *out, const uint16_t *gate, int ts, int m, int tid) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = (tid >> 5) + 16 * j;
            const unsigned off = (unsigned)((row < m ? row : m - 1) * ts + 4 * (tid & 31));
            y[j] = *reinterpret_cast<const Raw *>(out + off);
            gt[j] = stream_load8(gate + off);
        }
    }
    __device__ static float4 raw4(const uint4 &x) {
        return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w));
    }
    __device__ static float4 raw4(const uint2 &x) {
        return make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                           __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u));
    }
    __device__ void finish(OutT *out, int ts, const float *Os, int m, int tid, float4 w, float eps) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = (tid >> 5) + 16 * j, col = 4 * (tid & 31);
            const float4 x = *reinterpret_cast<const float4 *>(Os + ooff(row, col));
            const float4 r = raw4(y[j]);
            const float4 o = make_float4(r.x + x.x, r.y + x.y, r.z + x.z, r.w + x.w);
            float ss = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
#pragma unroll
            for (int k = 16; k >= 1; k >>= 1) ss += __shfl_xor(ss, k);
            const float inv = __builtin_amdgcn_rsqf(ss * (1.f / D) + eps);
            const float g0 = __uint_as_float(gt[j].x << 16), g1 = __uint_as_float(gt[j].x & 0xffff0000u);
            const float g2 = __uint_as_float(gt[j].y << 16), g3 = __uint_as_float(gt[j].y & 0xffff0000u);
            const float4 yv = make_float4(o.x * inv * w.x * sigmoid(g0), o.y * inv * w.y * sigmoid(g1),
                                          o.z * inv * w.z * sigmoid(g2), o.w * inv * w.w * sigmoid(g3));
            if (row < m) put4(out + (unsigned)(row * ts + col), yv);
        }
    }
};

// Two workgroups per CU: 128 registers per lane, and the Q tile shares its
// LDS with the staged output (66 KB per workgroup).
template <typename OutT, bool NG>
__global__ __launch_bounds__(NT, 4) void fix_kernel(PrefillArgs a, Segmented sp, float *ws, int nfinal) {
    __shared__ __attribute__((aligned(16))) __bf16 Sts[D * D];
    __shared__ __attribute__((aligned(16))) float Os[C * D];
    __shared__ long long first[kFixMaxPairs + 1];  // first chunk number of each pair
    __shared__ long long prows[kFixMaxPairs];       // rows corrected in each pair
    __bf16 *const Qs = reinterpret_cast<__bf16 *>(Os);

    const int tid = threadIdx.x;
    if ((int)blockIdx.x < nfinal) {  // final state of a local-start head
        const int uh = blockIdx.x / kFinalSlices;
        const float s2 = a.slopes[uh % a.heads] * LOG2E;
        if (!fix_head(s2, sp.seg_len, sp.fix_osz)) return;
        const int e = 4 * ((blockIdx.x % kFinalSlices) * NT + tid);
        float *u = sp.unit(ws, uh);
        const long long len = sequence_of(a, uh / a.heads).len;
        float4 acc = *reinterpret_cast<const float4 *>(sp.start_state(u, 0) + e);
        for (int g = 1; g < sp.used(len); ++g) {
            const float f = fast_exp2(-s2 * (float)seg_len_at(sp, len, g));
            const float4 x = *reinterpret_cast<const float4 *>(sp.start_state(u, g) + e);
            acc = make_float4(f * acc.x + x.x, f * acc.y + x.y, f * acc.z + x.z, f * acc.w + x.w);
        }
        *reinterpret_cast<float4 *>(a.state_out + (size_t)uh * D * D + e) = acc;
        return;
    }

    // rows and chunks per pair (none unless the head takes local starts; the
    // whole segment when its carried-in state is non-finite), then the chunks'
    // prefix sums (inclusive scan over the first kFixMaxPairs threads)
    const int gs = sp.segments - 1;
    const int pairs = a.units * a.heads * gs;
    long long x = 0;
    if (tid < pairs) {
        const int g = 1 + tid % gs, uh = tid / gs;
        const float s2 = a.slopes[uh % a.heads] * LOG2E;
        long long rows = 0;
        const long long len = seg_len_at(sp, sequence_of(a, uh / a.heads).len, g);
        if (len > 0 && fix_head(s2, sp.seg_len, sp.fix_osz))
            rows = start_poisoned(sp, sp.unit(ws, uh), g) ? len : fix_rows<NG>(s2, sp.seg_len, len);
        prows[tid] = rows;
        x = (rows + C - 1) / C;
    }
    for (int off = 1; off < kFixMaxPairs; off <<= 1) {
        if (tid < kFixMaxPairs) first[tid + 1] = x;
        __syncthreads();
        if (tid < kFixMaxPairs && tid >= off) x += first[tid + 1 - off];
        __syncthreads();
    }
    if (tid < kFixMaxPairs) first[tid + 1] = x;
    if (tid == 0) first[0] = 0;
    __syncthreads();

    // this workgroup's range: workgroups on one XCD (blockIdx % 8; nfinal and
    // the grid's remainder are multiples of 8) take consecutive ranges
    const long long total = uniform64(first[pairs]);
    const int nwg = gridDim.x - nfinal;
    const int r = (int)(blockIdx.x % 8) * (nwg / 8) + (int)(blockIdx.x - nfinal) / 8;
    const long long j0 = total * r / nwg, j1 = total * (r + 1) / nwg;
    if (j0 >= j1) return;

    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qh = w >> 2, cq = w & 3;
    const int ts = a.heads * D;  // 32-bit row offsets within a chunk (64 rows)
    auto load_q = [&](const FixChunk<OutT> &c, uint4 (&qx)[2], int th) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = (th >> 4) + 32 * i;
            qx[i] = stream_load16(c.q + (unsigned)((t < c.m ? t : c.m - 1) * ts + 8 * (th & 15)));
        }
    };
    using Rows = typename std::conditional<NG, NgRows<OutT>, OutRows<OutT>>::type;
    auto load_rows = [&](Rows &r, const FixChunk<OutT> &c, int th) {
        if constexpr (NG)
            r.load(c.o, c.gate, ts, c.m, th);
        else
            r.load(c.o, ts, c.m, th);
    };
    int p = 0;
    FixChunk<OutT> cur = fix_chunk<OutT, NG>(a, sp, first, prows, j0, p);
    uint4 qa[2];
    Rows ra;
    load_q(cur, qa, tid);
    load_rows(ra, cur, tid);
    int loaded = -1;
    for (long long j = j0; j < j1; ++j) {
        if (j > j0) __syncthreads();  // the previous chunk's reads of Os (= Qs) done
        // Lane-dependent offsets are recomputed from an opaque copy of the
        // thread index every chunk: hoisted out of the loop they would be
        // spilled, and a spill reload waits for every load in flight,
        // including the next chunk's.
        int tl = tid;
        asm volatile("" : "+v"(tl));
        const int ln = tl & 63;
        // the next chunk's loads go out before anything waits for this one's
        FixChunk<OutT> nxt = cur;
        uint4 qb[2] = {qa[0], qa[1]};
        Rows rb = ra;
        if (j + 1 < j1) {
            nxt = fix_chunk<OutT, NG>(a, sp, first, prows, j + 1, p);
            load_q(nxt, qb, tl);
            load_rows(rb, nxt, tl);
        }
        if (cur.pair != loaded) {
            // S_in(g) of this pair as bf16 S^T: the thread with value column
            // c and key quad kq forms S_in[4(kq + 4i) + r + 64 half][c], i < 4,
            // r < 4, half < 2 (the previous chunk's reads of Sts ended before
            // its second barrier)
            const int c = tl & (D - 1), kq = tl >> 7;
            float *u = sp.unit(ws, cur.uh);
#pragma unroll
            for (int half = 0; half < 2; ++half) {  // 16 elements at a time (registers)
                float acc[4][4];
                {
                    const float *e = sp.start_state(u, 0) + (4 * kq + 64 * half) * D + c;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[i][r] = e[(16 * i + r) * D];
                }
                for (int g = 1; g < cur.g; ++g) {  // segments before cur.g are whole
                    const float f = fast_exp2(-cur.s2 * (float)sp.seg_len);
                    const float *e = sp.start_state(u, g) + (4 * kq + 64 * half) * D + c;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[i][r] = f * acc[i][r] + e[(16 * i + r) * D];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bf16x4 x;
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[r] = static_cast<__bf16>(acc[i][r]);
                    *reinterpret_cast<bf16x4 *>(Sts + L128::off(c, 4 * (kq + 4 * i) + 64 * half)) = x;
                }
            }
            loaded = cur.pair;
        }
        // this chunk's q rows into the tile (rows past m zeroed)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = (tl >> 4) + 32 * i;
            *reinterpret_cast<uint4 *>(Qs + L128::off(t, 8 * (tl & 15))) = keep_if(t < cur.m, qa[i]);
        }
        __syncthreads();  // Q tile and S^T visible
        f32x16 o;
#pragma unroll
        for (int v = 0; v < 16; ++v) o[v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            o = mma(ld_op<L128>(Sts, 32 * cq, 16 * ks, ln), ld_op<L128>(Qs, 32 * qh, 16 * ks, ln), o);
        o *= fast_exp2(-cur.s2 * (float)(cur.t0 + 32 * qh + (ln & 31) + 1));
        __syncthreads();  // every read of Qs and Sts done
        stage_out(Os, o, qh, cq, ln);
        __syncthreads();  // Os visible
        if constexpr (NG)
            ra.finish(cur.o, ts, Os, cur.m, tl,
                      *reinterpret_cast<const float4 *>(a.ng.norm_weight + cur.h * D + 4 * (tl & 31)), a.ng.eps);
        else
            ra.add_store(cur.o, ts, Os, cur.m, tl);
        cur = nxt;
        qa[0] = qb[0];
        qa[1] = qb[1];
        ra = rb;
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
    // heads may take local-start segments; the correction's extra traffic per
    // token is, in units of 256 B, 1 + sizeof(OutT): q read and the output row
    // read and written (with the norm-gate epilogue the gate is read by the
    // correction pass instead of the main pass)
    const int fix_osz = p.segments > 1 ? (int)sizeof(OutT) : 0;
    const Segmented sp{p.segments, p.pieces, p.seg_len, p.piece_len, fix_osz};
    if (p.segments > 1) {
        hipLaunchKernelGGL(piece_state_kernel, dim3((unsigned)(uh * p.pieces)), dim3(NT), 0, stream,
                           a, sp, ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(uh * kCombineSlices)), dim3(kCombineThreads),
                           0, stream, a.slopes, a.heads, a.state_in, a.state_in_t, sp,
                           SeqLens{a.cu_seqlens, a.total_tokens, a.seqlen}, ws);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.ng.gate)
        hipLaunchKernelGGL((head_kernel<OutT, true>), dim3((unsigned)(uh * p.segments)), dim3(NT), 0,
                           stream, a, sp, ws);
    else
        hipLaunchKernelGGL((head_kernel<OutT, false>), dim3((unsigned)(uh * p.segments)), dim3(NT), 0,
                           stream, a, sp, ws);
    if (!fix_osz) return hipGetLastError();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (uh * (p.segments - 1) > kFixMaxPairs) return hipErrorInvalidValue;  // not a segmented plan
    const int nfinal = a.state_out ? (int)(uh * kFinalSlices) : 0;
    if (a.ng.gate)
        hipLaunchKernelGGL((fix_kernel<OutT, true>), dim3((unsigned)(nfinal + kFixWorkgroups)), dim3(NT), 0, stream,
                           a, sp, ws, nfinal);
    else
        hipLaunchKernelGGL((fix_kernel<OutT, false>), dim3((unsigned)(nfinal + kFixWorkgroups)), dim3(NT), 0, stream,
                           a, sp, ws, nfinal);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_heads(const PrefillArgs &a, const PrefillPlan &plan, void *workspace,
                                lt_dtype out_dtype, hipStream_t stream) {
    return out_dtype == LT_F32 ? launch<float>(a, plan, workspace, stream)
                               : launch<__bf16>(a, plan, workspace, stream);
}

}  // namespace lt
