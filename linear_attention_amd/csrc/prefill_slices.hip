// Lightning Attention prefill for gfx950 (MI355X).
//
// Operator: MiniMax Signal Lab · M1, §03 Lightning Attention. Per head, with a
// d x d fp32 state S carried across blocks:
//   O_t = [(Q_t K_t^T) ⊙ D] V_t + (Q_t ⊙ d_q) S_{t-1}
//   S_t = e^{-s m} S_{t-1} + (K_t ⊙ d_k)^T V_t
// with D_ij = e^{-s(i-j)}[i>=j], d_q[i] = e^{-s i}, d_k[j] = e^{-s(m-j)} for a
// block of m tokens (positions 1..m).
//
// Design (gfx950-first, not the pages' GPU design):
//  * Work unit = (sequence, head, 32-column slice of the value dimension).
//    Output columns J depend only on V[:, J] and S[:, J], so the four slices of
//    a head are fully independent: no cross-workgroup scan, no workspace, and
//    batch-1 prefill still fills 256 CUs with 64 heads. Q and K are re-read by
//    the four slices; the launch maps the four slices of a head to one XCD so
//    those re-reads hit that XCD's L2 and HBM sees each byte once.
//  * Blocks are evaluated as 64-token sub-blocks (one per loop iteration). Any
//    block length gives the same operator value (the block form re-associates
//    the per-token recurrence exactly), and 64 keeps every tile of a 4-wave
//    workgroup in LDS with room for two workgroups per CU.
//  * All four products run on MFMA (bf16 16x16x32 with fp32 accumulation for
//    bf16 inputs; fp32 16x16x4 for fp32 inputs):
//      scores^T = K Q^T                      (keys x queries; causal tiles only)
//      O^T      = S^T (Q ⊙ d_q)^T + V^T P^T  (value cols x queries)
//      dS       = (K ⊙ d_k)^T V              (key dim x value cols)
//    The scores are produced in the exact register layout the P operand of
//    V^T P^T needs, so P never goes through LDS. The state stays in the MFMA
//    accumulators of the four waves for the whole sequence; each sub-block it
//    is also written once to LDS (rounded to the MFMA input type) as the
//    operand of the next sub-block's inter-block product.
//  * Decay factors are computed in registers with exp2 of non-positive
//    arguments only (never e^{+s j}, which would overflow fp32 for large s).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "internal.h"

namespace lt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int D = kHeadDim;         // 128
constexpr int C = 64;               // tokens per sub-block
constexpr int NSL = kValueSlices;   // value slices per head
constexpr int SL = D / NSL;         // 32 value columns per workgroup
constexpr int NT = 256;             // threads per workgroup (4 waves)
constexpr float LOG2E = 1.4426950408889634f;

static_assert(SL == 32 && C == 64 && D == 128, "tile shapes are fixed below");

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Component-wise select (keeps vector selects in registers).
__device__ __forceinline__ uint4 keep_if(bool keep, uint4 x) {
    return make_uint4(keep ? x.x : 0u, keep ? x.y : 0u, keep ? x.z : 0u, keep ? x.w : 0u);
}
__device__ __forceinline__ float4 keep_if(bool keep, float4 x) {
    return make_float4(keep ? x.x : 0.f, keep ? x.y : 0.f, keep ? x.z : 0.f, keep ? x.w : 0.f);
}

// 2^x with the hardware exp2 (v_exp_f32, about 1 ulp). Arguments here are
// never positive; results below the fp32 normal range may flush to zero, which
// changes a decay product by less than 2^-126 relative.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Per-input-type MFMA policy. Operands are read from LDS rows in which the
// contraction index is contiguous; lane l reads row (l % 16), contraction
// slots [KPL*(l/16), KPL*(l/16)+KPL) of each KSTEP-wide step.
template <typename T> struct Mma;

template <> struct Mma<__bf16> {
    using E = __bf16;
    using Frag = bf16x8;
    static constexpr int KSTEP = 32;
    static constexpr int KPL = 8;
    static constexpr int PAD = 8;      // 16-byte row padding against bank conflicts
    static constexpr int VEC = 8;      // elements per 16-byte global load
    __device__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static Frag ld(const E *p) { return *reinterpret_cast<const Frag *>(p); }
    __device__ static float to_f32(uint32_t bits16) { return bf16_bits_to_f32(bits16); }
};

template <> struct Mma<float> {
    using E = float;
    using Frag = float;
    static constexpr int KSTEP = 4;
    static constexpr int KPL = 1;
    static constexpr int PAD = 4;
    static constexpr int VEC = 4;
    __device__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ static Frag ld(const E *p) { return *p; }
};

// acc += A[16 rows][K] * B[K][16 cols], A rows and B columns K-contiguous in LDS.
template <typename M, int K>
__device__ __forceinline__ f32x4 contract(f32x4 acc, const typename M::E *a, int a_pitch,
                                          const typename M::E *b, int b_pitch, int lane) {
    const typename M::E *pa = a + (lane & 15) * a_pitch + (lane >> 4) * M::KPL;
    const typename M::E *pb = b + (lane & 15) * b_pitch + (lane >> 4) * M::KPL;
#pragma unroll
    for (int ks = 0; ks < K / M::KSTEP; ++ks)
        acc = M::mma(M::ld(pa + ks * M::KSTEP), M::ld(pb + ks * M::KSTEP), acc);
    return acc;
}

// acc[j] += A_j[16 rows][K] * B_j[K][16 cols] for N independent tiles; the
// contraction loop is outermost so the N MFMA chains interleave.
// a(j) and b(j) return the first row of tile j's A and B operands.
template <typename M, int K, int N, typename FA, typename FB>
__device__ __forceinline__ void contract_n(f32x4 (&acc)[N], FA a, FB b, int a_pitch, int b_pitch,
                                           int lane) {
    const int oa = (lane & 15) * a_pitch + (lane >> 4) * M::KPL;
    const int ob = (lane & 15) * b_pitch + (lane >> 4) * M::KPL;
#pragma unroll
    for (int ks = 0; ks < K / M::KSTEP; ++ks)
#pragma unroll
        for (int j = 0; j < N; ++j)
            acc[j] = M::mma(M::ld(a(j) + oa + ks * M::KSTEP), M::ld(b(j) + ob + ks * M::KSTEP),
                            acc[j]);
}

// O^T[cols][queries] += V^T[cols][keys] P^T[keys][queries] over the sub-block's
// four key tiles (P is zero above the diagonal). sc[kt] holds scores^T tile kt
// in accumulator layout:
// lane l has keys 16kt + 4(l/16) + r, r = 0..3, for query (l % 16).
template <typename M>
__device__ __forceinline__ void intra(f32x4 (&o)[2], const f32x4 (&sc)[4],
                                      const typename M::E *vts, int tp, int lane);

template <>
__device__ __forceinline__ void intra<Mma<__bf16>>(f32x4 (&o)[2], const f32x4 (&sc)[4],
                                                   const __bf16 *vts, int tp, int lane) {
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        // contraction slots 0..3 -> keys 32ks + 4g + r, slots 4..7 -> keys 32ks + 16 + 4g + r
        bf16x8 b;
        const f32x4 lo = sc[2 * ks];
        const f32x4 hi = sc[2 * ks + 1];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            b[r] = static_cast<__bf16>(lo[r]);
            b[4 + r] = static_cast<__bf16>(hi[r]);
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const __bf16 *row = vts + (16 * ct + li) * tp + 32 * ks + 4 * g;
            const bf16x4 a0 = *reinterpret_cast<const bf16x4 *>(row);
            const bf16x4 a1 = *reinterpret_cast<const bf16x4 *>(row + 16);
            bf16x8 a;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                a[r] = a0[r];
                a[4 + r] = a1[r];
            }
            o[ct] = Mma<__bf16>::mma(a, b, o[ct]);
        }
    }
}

template <>
__device__ __forceinline__ void intra<Mma<float>>(f32x4 (&o)[2], const f32x4 (&sc)[4],
                                                  const float *vts, int tp, int lane) {
    const int li = lane & 15, g = lane >> 4;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                o[ct] = Mma<float>::mma(vts[(16 * ct + li) * tp + 16 * kt + 4 * g + r], sc[kt][r],
                                        o[ct]);
    }
}

// ---- global -> register staging of one sub-block ---------------------------
// bf16: each thread holds 4 consecutive tokens x 8 key/query dims of Q and K
//       (tokens 4*(tid/16) + i, dims 8*(tid%16) + e), and 1 token x 8 value
//       columns of the slice (token tid/4, columns 8*(tid%4) + e).
// fp32: 8 consecutive tokens x 4 dims of Q and K (tokens 8*(tid/32) + i, dims
//       4*(tid%32) + e), and 2 tokens x 4 columns (tokens tid/8 + 32 i,
//       columns 4*(tid%8) + e).
template <typename T> struct Stage;

template <> struct Stage<__bf16> {
    static constexpr int TPT = 4, NV = 1;
    uint4 q[TPT], k[TPT], v[NV];

    // Every thread issues the same loads on every call (row indices clamped
    // into [0, m)), so the number of memory operations in flight never depends
    // on m and the compiler can count them exactly. Rows t >= m are zeroed in
    // store(), not here, so nothing waits on these loads before the data is
    // needed. `ts` (elements between tokens) times 63 fits in 32 bits.
    __device__ void load(const uint16_t *qg, const uint16_t *kg, const uint16_t *vg, int ts, int m,
                         int tid) {
        const int seg = tid & 15, t0 = 4 * (tid >> 4);
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const int t = t0 + i;
            const int row = (t < m ? t : m - 1) * ts + 8 * seg;
            q[i] = *reinterpret_cast<const uint4 *>(qg + row);
            k[i] = *reinterpret_cast<const uint4 *>(kg + row);
        }
        const int vt = tid >> 2, vs = tid & 3;
        v[0] = *reinterpret_cast<const uint4 *>(vg + (vt < m ? vt : m - 1) * ts + 8 * vs);
    }

    // Writes Q, K (row-major), K ⊙ d_k transposed, and V transposed into LDS.
    __device__ void store(__bf16 *Qs, __bf16 *Ks, __bf16 *Kts, __bf16 *Vts, int qp, int tp, int m,
                          float s2, int tid) {
        const int seg = tid & 15, t0 = 4 * (tid >> 4);
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            q[i] = keep_if(t0 + i < m, q[i]);
            k[i] = keep_if(t0 + i < m, k[i]);
            *reinterpret_cast<uint4 *>(Qs + (t0 + i) * qp + 8 * seg) = q[i];
            *reinterpret_cast<uint4 *>(Ks + (t0 + i) * qp + 8 * seg) = k[i];
        }
        v[0] = keep_if((tid >> 2) < m, v[0]);
        float dk[TPT];
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const int t = t0 + i;
            dk[i] = (t < m) ? fast_exp2(-s2 * (float)(m - 1 - t)) : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x4 col;
#pragma unroll
            for (int i = 0; i < TPT; ++i) {
                const uint32_t word = (&k[i].x)[e >> 1];
                const uint32_t bits = (e & 1) ? (word >> 16) : (word & 0xffffu);
                col[i] = static_cast<__bf16>(bf16_bits_to_f32(bits) * dk[i]);
            }
            *reinterpret_cast<bf16x4 *>(Kts + (8 * seg + e) * tp + t0) = col;
        }
        const int vt = tid >> 2, vs = tid & 3;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t word = (&v[0].x)[e >> 1];
            const uint16_t bits = (e & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xffffu);
            reinterpret_cast<uint16_t *>(Vts)[(8 * vs + e) * tp + vt] = bits;
        }
    }
};

template <> struct Stage<float> {
    static constexpr int TPT = 8, NV = 2;
    float4 q[TPT], k[TPT], v[NV];

    __device__ void load(const float *qg, const float *kg, const float *vg, int ts, int m, int tid) {
        const int seg = tid & 31, t0 = 8 * (tid >> 5);
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const int t = t0 + i;
            const int row = (t < m ? t : m - 1) * ts + 4 * seg;
            q[i] = *reinterpret_cast<const float4 *>(qg + row);
            k[i] = *reinterpret_cast<const float4 *>(kg + row);
        }
        const int vs = tid & 7;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int vt = (tid >> 3) + 32 * j;
            v[j] = *reinterpret_cast<const float4 *>(vg + (vt < m ? vt : m - 1) * ts + 4 * vs);
        }
    }

    __device__ void store(float *Qs, float *Ks, float *Kts, float *Vts, int qp, int tp, int m,
                          float s2, int tid) {
        const int seg = tid & 31, t0 = 8 * (tid >> 5);
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            q[i] = keep_if(t0 + i < m, q[i]);
            k[i] = keep_if(t0 + i < m, k[i]);
            *reinterpret_cast<float4 *>(Qs + (t0 + i) * qp + 4 * seg) = q[i];
            *reinterpret_cast<float4 *>(Ks + (t0 + i) * qp + 4 * seg) = k[i];
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j] = keep_if((tid >> 3) + 32 * j < m, v[j]);
        float dk[TPT];
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const int t = t0 + i;
            dk[i] = (t < m) ? fast_exp2(-s2 * (float)(m - 1 - t)) : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float col[TPT];
#pragma unroll
            for (int i = 0; i < TPT; ++i) col[i] = (&k[i].x)[e] * dk[i];
            float4 *dst = reinterpret_cast<float4 *>(Kts + (4 * seg + e) * tp + t0);
            dst[0] = make_float4(col[0], col[1], col[2], col[3]);
            dst[1] = make_float4(col[4], col[5], col[6], col[7]);
        }
        const int vs = tid & 7;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int vt = (tid >> 3) + 32 * j;
#pragma unroll
            for (int e = 0; e < 4; ++e) Vts[(4 * vs + e) * tp + vt] = (&v[j].x)[e];
        }
    }
};

template <typename T> struct Storage { using type = T; };
template <> struct Storage<__bf16> { using type = uint16_t; };

__device__ __forceinline__ void store_out(float *p, f32x4 x) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store_out(__bf16 *p, f32x4 x) {
    bf16x4 y;
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = static_cast<__bf16>(x[r]);
    *reinterpret_cast<bf16x4 *>(p) = y;
}

template <typename InT, typename OutT>
__global__ __launch_bounds__(NT) void prefill_kernel(PrefillArgs a) {
    using M = Mma<InT>;
    using E = typename M::E;
    using G = typename Storage<InT>::type;   // global element type
    constexpr int QP = D + M::PAD;           // pitch of Qs, Ks, Sts rows
    constexpr int TP = C + M::PAD;           // pitch of Kts, Vts rows
    __shared__ __attribute__((aligned(16))) E Qs[C * QP];
    __shared__ __attribute__((aligned(16))) E Ks[C * QP];
    __shared__ __attribute__((aligned(16))) E Kts[D * TP];
    __shared__ __attribute__((aligned(16))) E Vts[SL * TP];
    __shared__ __attribute__((aligned(16))) E Sts[2][SL * QP];

    // XCD-aware work mapping: the hardware deals workgroups round-robin over the
    // 8 XCDs, so virtual id v = (bid % 8) * (nwg / 8) + bid / 8 gives each XCD a
    // contiguous run of v, and the NSL slices of a head share one XCD's L2.
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int vid = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
    const int slice = vid % NSL;
    const int uh = vid / NSL;
    const int h = uh % a.heads;
    const int n = uh / a.heads;

    long long start, len;
    if (a.cu_seqlens) {
        const long long T = a.total_tokens;
        long long lo = a.cu_seqlens[n], hi = a.cu_seqlens[n + 1];
        lo = lo < 0 ? 0 : (lo > T ? T : lo);
        hi = hi < lo ? lo : (hi > T ? T : hi);
        start = lo;
        len = hi - lo;
    } else {
        start = (long long)n * a.seqlen;
        len = a.seqlen;
    }

    const int ts = a.heads * D;  // elements between consecutive tokens (checked < 2^24)
    const long long base = (start * a.heads + h) * D;
    const G *qg = static_cast<const G *>(a.q) + base;
    const G *kg = static_cast<const G *>(a.k) + base;
    const G *vg = static_cast<const G *>(a.v) + base + slice * SL;
    OutT *og = static_cast<OutT *>(a.o) + base + slice * SL;

    const float s2 = a.slopes[h] * LOG2E;
    const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform

    // State slice S[key][32 value columns]: wave w keeps keys 32w + 16rt + 4g + r,
    // columns 16ct + li, in MFMA accumulator layout.
    f32x4 S[2][2];
    const long long sbase = ((long long)n * a.heads + h) * D * D + slice * SL;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[rt][ct][r] = a.state_in ? a.state_in[sbase + (32 * w + 16 * rt + 4 * g + r) * D +
                                                       16 * ct + li]
                                          : 0.f;

    auto write_state_operand = [&](E *dst) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                store_out(dst + (16 * ct + li) * QP + 32 * w + 16 * rt + 4 * g, S[rt][ct]);
            }
    };
    write_state_operand(Sts[0]);

    Stage<InT> stage;
    const long long nfull = len / C;               // full sub-blocks
    const int tail = (int)(len - nfull * C);        // tokens in a last short one
    const long long nchunks = nfull + (tail > 0);
    auto chunk_len = [&](long long c) { return c < nfull ? C : tail; };
    if (nchunks > 0) stage.load(qg, kg, vg, ts, chunk_len(0), tid);

    const int qpos = 16 * w + li;  // query row (in the sub-block) of this lane's outputs
    int cur = 0;
    // Outputs of a full sub-block are stored one step late, after the wait for
    // the next tiles and before the next prefetch is issued: the prefetch loads
    // are then always the newest memory operations in flight, so waiting for
    // them never waits on output stores issued after them.
    f32x4 o_prev[2];
    OutT *orow_prev = og;
    auto flush = [&]() {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) store_out(orow_prev + 16 * ct + 4 * g, o_prev[ct]);
    };
    // One sub-block of m tokens. FULL sub-blocks (m == C) have no data-dependent
    // branch around any memory operation.
    auto step = [&](long long c, int m, bool have_prev, auto full) {
        constexpr bool FULL = decltype(full)::value;
        __syncthreads();  // previous sub-block's readers of the tiles are done
        stage.store(Qs, Ks, Kts, Vts, QP, TP, m, s2, tid);
        if (have_prev) flush();
        if (FULL) {
            // prefetch the next sub-block (after the last one, re-read this one)
            const long long cn = (c + 1 < nchunks) ? c + 1 : c;
            const long long off = cn * C * (long long)ts;
            stage.load(qg + off, kg + off, vg + off, ts, chunk_len(cn), tid);
        }
        __syncthreads();  // tiles and the previous state operand are visible

        // scores^T tiles (keys 16kt.., queries 16w..) and the inter-block product
        // S^T Q^T share the B operand (this wave's 16 queries): six independent
        // MFMA chains, interleaved.
        f32x4 acc[6];
        const E *sts = Sts[cur];
        const E *qrow = Qs + 16 * w * QP;
#pragma unroll
        for (int j = 0; j < 6; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        contract_n<M, D, 6>(
            acc, [&](int j) { return j < 4 ? Ks + 16 * j * QP : sts + 16 * (j - 4) * QP; },
            [&](int) { return qrow; }, QP, QP, lane);

        f32x4 sc[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int diff = qpos - (16 * kt + 4 * g + r);
                sc[kt][r] = diff >= 0 ? acc[kt][r] * fast_exp2(-s2 * (float)diff) : 0.f;
            }

        // O^T = S^T (Q ⊙ d_q)^T + V^T P^T for value columns 16ct.., queries 16w..
        const float dq = fast_exp2(-s2 * (float)(qpos + 1));
        o_prev[0] = acc[4] * dq;
        o_prev[1] = acc[5] * dq;
        intra<M>(o_prev, sc, Vts, TP, lane);
        orow_prev = og + (c * C + qpos) * (long long)ts;
        if (!FULL && qpos < m) flush();

        // S = e^{-s m} S + (K ⊙ d_k)^T V   (keys 32w.., all 32 columns)
        const float bd = fast_exp2(-s2 * (float)m);
        f32x4 sacc[4] = {S[0][0] * bd, S[0][1] * bd, S[1][0] * bd, S[1][1] * bd};
        contract_n<M, C, 4>(
            sacc, [&](int j) { return Kts + (32 * w + 16 * (j >> 1)) * TP; },
            [&](int j) { return Vts + 16 * (j & 1) * TP; }, TP, TP, lane);
        S[0][0] = sacc[0];
        S[0][1] = sacc[1];
        S[1][0] = sacc[2];
        S[1][1] = sacc[3];
        cur ^= 1;
        write_state_operand(Sts[cur]);
    };
    if (nfull > 0) step(0, C, false, std::true_type{});
    for (long long c = 1; c < nfull; ++c) step(c, C, true, std::true_type{});
    if (tail > 0)
        step(nfull, tail, nfull > 0, std::false_type{});
    else if (nfull > 0)
        flush();

    if (a.state_out) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    a.state_out[sbase + (32 * w + 16 * rt + 4 * g + r) * D + 16 * ct + li] =
                        S[rt][ct][r];
    }
}

template <typename InT, typename OutT>
hipError_t launch(const PrefillArgs &a, hipStream_t stream) {
    clear_pending_error();
    const long long nwg = (long long)a.units * a.heads * NSL;
    hipLaunchKernelGGL((prefill_kernel<InT, OutT>), dim3((unsigned)nwg), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t load_prefill_slices_code() {
    hipFuncAttributes attr;
    return hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(&prefill_kernel<__bf16, float>));
}

hipError_t launch_prefill_slices(const PrefillArgs &a, lt_dtype in_dtype, lt_dtype out_dtype,
                          hipStream_t stream) {
    if (in_dtype == LT_BF16)
        return out_dtype == LT_F32 ? launch<__bf16, float>(a, stream) : launch<__bf16, __bf16>(a, stream);
    return out_dtype == LT_F32 ? launch<float, float>(a, stream) : launch<float, __bf16>(a, stream);
}

}  // namespace lt
