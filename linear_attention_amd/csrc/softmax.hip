// Softmax attention of the hybrid's other layers on gfx950 (MI355X): causal,
// grouped K/V heads, rotary position embedding on part of the head.
//
// MiniMax Signal Lab · M1, §02: the softmax layers project 64 query heads of
// 128 and 8 K/V heads of 128, and only they apply RoPE, on 64 of the 128
// dimensions. Per query head h (K/V head g = h / (Hq / Hkv)), token t at
// position pos0 + t:
//   o_t = sum_{j <= t} softmax_j(scale * rope(q_t) . rope(k_j)) v_j
// RoPE pairs feature m with m + R/2 (m < R/2, R = rope dims) and rotates the
// pair by position * base^(-2m/R); angles are formed in fp64 and reduced mod
// 2 pi before the fp32 sine and cosine, so they stay exact at 1M positions.
//
// Prefill (flash-attention forward):
//  * rope_rows_kernel writes rope(k) once (bf16, workspace);
//  * one 8-wave workgroup per (sequence, K/V head, block of queries): its waves
//    cover hpw = gcd(group size, 8) query heads of that K/V head's group and
//    8 / hpw consecutive 32-query blocks, so each K/V tile staged in LDS feeds
//    all eight waves (FaGeom below); a wave's 32 queries are held as MFMA
//    operands in registers (rope applied, scaled by scale * log2(e)); per
//    64-key block S^T = K Q^T on v_mfma_f32_32x32x16_bf16, accumulated onto
//    the negated reference maximum (a lane owns one query and 32 keys, so the
//    test for a move of the maximum and the sum are lane-local; a move takes
//    one xor-32 shuffle); the probabilities stay in registers as the B operand
//    of O^T += V^T P^T; blocks past a wave's last query are skipped; heavy (late)
//    query blocks are launched first, and the workgroups of one
//    (sequence, K/V head) run on one XCD.
// Decode: rope_append_kernel writes rope(k_new), v_new into the KV cache; then
// one wave per (sequence, K/V head, key split) serves the group's query heads
// as MFMA columns (S^T = K Q^T, O^T += V^T P^T over 32-key blocks staged in
// the wave's own LDS tiles), and a combine kernel merges the splits' partial
// softmax states (flash-decoding).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <numeric>
#include <type_traits>
#include <utility>

#include "internal.h"
#include "tiles.h"

namespace lt {
namespace {

constexpr int SKB = 64;       // keys per block
constexpr int SNT = 256;      // 4 waves (RoPE and decode kernels)
constexpr int FNT = 512;      // 8 waves (prefill)
constexpr int FW = FNT / 64;
// LDS tile pitches (bf16). K rows are read whole (ds_read_b128 per lane, a lane
// per row): a pitch of 68 dwords puts 16 consecutive rows on distinct banks. V
// is read with ds_read_b64_tr_b16 (four rows per 16-lane group): a pitch of
// 80 dwords (16 mod 64) keeps the four rows of both 16-lane groups of a half
// wave on distinct banks.
constexpr int SPT = D + 8;
constexpr int SPV = D + 32;
using LK = LPad<SPT>;
using LV = LPad<SPV>;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.f, (__bf16)1.f};
// Growth of a score over the running reference maximum (log2 units) that is
// let pass before O and l are rescaled.
constexpr float kStale = 8.f;

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {
    const __bf16 b = static_cast<__bf16>(f);
    uint16_t u;
    __builtin_memcpy(&u, &b, 2);
    return u;
}

// V^T operand for O^T += V^T P^T with P^T taken straight from the S^T
// accumulators: lane l gets V[k0 + 4(l/32) + e][c0 + l%32] for e = 0..3 and
// V[k0 + 8 + 4(l/32) + e - 4][c0 + l%32] for e = 4..7 (the key order in which
// the accumulator layout holds a lane's scores; the contraction does not care
// about the order as long as both operands share it).
__device__ __forceinline__ bf16x8 ld_vt(const __bf16 *t, int c0, int k0, int lane) {
    const int li = lane & 15, grp = lane >> 4;
    const int row = k0 + 4 * (grp >> 1) + (li >> 2), col = c0 + 16 * (grp & 1) + 4 * (li & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(t + LV::off(row, col)));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(t + LV::off(row + 8, col)));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Rotation rates of the R/2 feature pairs, base^(-2m/R) in turns (fp64),
// into th[0 .. R/2) of the workgroup's LDS: one fp64 exp2 per thread at most,
// instead of one per rotated element. The caller synchronises the workgroup
// before reading the table.
constexpr int kRopePairs = D / 2;
__device__ __forceinline__ void rope_table(double *th, int R, double log2_base, int tid, int nthreads) {
    for (int m = tid; m < R / 2; m += nthreads)
        th[m] = exp2(-(2.0 * m / R) * log2_base) * 0.15915494309189535;
}

// sin and cos of position * rate (rate in turns): the angle is formed in fp64
// as a fraction of a turn and reduced to [0, 1) before the hardware sine and
// cosine (which take turns), so it stays exact at any position.
__device__ __forceinline__ void rope_sincos(long long pos, double th, float &s, float &c) {
    double t = (double)pos * th;
    t -= floor(t);
    s = __builtin_amdgcn_sinf((float)t);
    c = __builtin_amdgcn_cosf((float)t);
}

// rope(x) of one row of d bf16 features into y: thread j < 16 handles features
// 8j..8j+7; a thread in the first half of the rotated span also writes the
// partner features.
__device__ __forceinline__ void rope_row(const uint16_t *x, uint16_t *y, long long pos, int R,
                                         const double *th, int j) {
    const int f0 = 8 * j;
    const int half = R / 2;
    if (f0 >= half && f0 < R) return;  // written by the partner thread
    uint16_t a[8];
    *reinterpret_cast<uint4 *>(a) = *reinterpret_cast<const uint4 *>(x + f0);
    if (f0 >= R) {  // not rotated
        *reinterpret_cast<uint4 *>(y + f0) = *reinterpret_cast<const uint4 *>(a);
        return;
    }
    uint16_t b[8], ra[8], rb[8];
    *reinterpret_cast<uint4 *>(b) = *reinterpret_cast<const uint4 *>(x + f0 + half);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float s, c;
        rope_sincos(pos, th[f0 + e], s, c);
        const float u = bf2f(a[e]), w = bf2f(b[e]);
        ra[e] = f2bf(u * c - w * s);
        rb[e] = f2bf(u * s + w * c);
    }
    *reinterpret_cast<uint4 *>(y + f0) = *reinterpret_cast<const uint4 *>(ra);
    *reinterpret_cast<uint4 *>(y + f0 + half) = *reinterpret_cast<const uint4 *>(rb);
}

// One query row as the 8 B operands of S^T = K Q^T: operand ks of lane half hf
// holds features 16ks + 8hf + e, e = 0..7, after rope at position pos, times
// qs (the score scale with log2(e) folded in, so softmax runs on exp2).
__device__ __forceinline__ void load_q_operand(const uint16_t *qg, long long pos, int rope_dims,
                                               const double *th, float qs, int hf,
                                               bf16x8 (&qop)[D / 16]) {
    float x[D / 16][8];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        uint16_t u[8];
        *reinterpret_cast<uint4 *>(u) = *reinterpret_cast<const uint4 *>(qg + 16 * ks + 8 * hf);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[ks][e] = bf2f(u[e]);
    }
    // rotate-half pairs lie hs = rope_dims/32 operand steps apart; feature
    // 16ks + 8hf + e is in the first half of the rotated span iff ks < hs
    const int hs = rope_dims / 32;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int dd = 1; dd <= D / 32; ++dd)
            if (ks + dd < D / 16 && dd == hs && ks < hs) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float s, c;
                    rope_sincos(pos, th[16 * ks + 8 * hf + e], s, c);
                    const float u = x[ks][e], v = x[ks + dd][e];
                    x[ks][e] = u * c - v * s;
                    x[ks + dd][e] = u * s + v * c;
                }
            }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qop[ks][e] = static_cast<__bf16>(x[ks][e] * qs);
}

// rope of every k row: [B, L, Hkv, d] -> same shape. 16 threads per row.
__global__ __launch_bounds__(SNT) void rope_rows_kernel(SoftmaxArgs a, uint16_t *kr) {
    __shared__ double th[kRopePairs];
    rope_table(th, a.rope_dims, a.log2_base, threadIdx.x, SNT);
    __syncthreads();
    const long long row = (long long)blockIdx.x * (SNT / 16) + threadIdx.x / 16;
    const long long rows = (long long)a.batch * a.seqlen * a.kv_heads;
    if (row >= rows) return;
    const long long t = (row / a.kv_heads) % a.seqlen;
    rope_row(static_cast<const uint16_t *>(a.k) + row * D, kr + row * D, a.pos0 + t, a.rope_dims, th,
             threadIdx.x % 16);
}

template <typename OutT>
__device__ __forceinline__ void put_out4(OutT *p, float x, float y, float z, float w);
template <>
__device__ __forceinline__ void put_out4<float>(float *p, float x, float y, float z, float w) {
    stream_store(p, make_float4(x, y, z, w));
}
template <>
__device__ __forceinline__ void put_out4<__bf16>(__bf16 *p, float x, float y, float z, float w) {
    const bf16x4 b = {static_cast<__bf16>(x), static_cast<__bf16>(y), static_cast<__bf16>(z),
                      static_cast<__bf16>(w)};
    stream_store_bits(p, b);
}

// Workgroup geometry of the prefill kernel: FW waves of 32 queries each cover
// hpw query heads of one K/V group (hpw = gcd(group size, FW)) and
// FW / hpw consecutive 32-query blocks, so every K/V tile staged in LDS feeds
// FW waves. Workgroups are numbered so that the ones of one (sequence, K/V
// head) run on one XCD (the hardware deals workgroups to the 8 XCDs in turn),
// where that head's K and V stay in the XCD's L2; within a group the late
// (long) query blocks come first.
struct FaGeom {
    int hpw;         // query heads per workgroup
    int qpw;         // queries per workgroup (32 * FW / hpw)
    int nqb;         // query blocks per head
    int per_group;   // workgroups per (sequence, K/V head)
    long long real;  // workgroups with work (grid is this rounded up to 8)
};

template <typename OutT>
__global__ __launch_bounds__(FNT) void fa_prefill_kernel(SoftmaxArgs a, const uint16_t *kr, FaGeom geo) {
    __shared__ __attribute__((aligned(16))) __bf16 Ks[2][SKB * SPT];
    __shared__ __attribute__((aligned(16))) __bf16 Vs[2][SKB * SPV];
    __shared__ double th[kRopePairs];

    const long long per_xcd = gridDim.x / 8;
    const long long u = (long long)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (u >= geo.real) return;  // padding workgroup (the whole workgroup leaves)
    rope_table(th, a.rope_dims, a.log2_base, threadIdx.x, FNT);
    __syncthreads();
    const int G = a.q_heads / a.kv_heads;
    const int bg = (int)(u / geo.per_group), rem = (int)(u % geo.per_group);
    const int hsubs = G / geo.hpw;
    const int qb = geo.nqb - 1 - rem / hsubs;  // late blocks first
    const int b = bg / a.kv_heads, g = bg % a.kv_heads;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = g * G + (rem % hsubs) * geo.hpw + w % geo.hpw;
    const int r32 = lane & 31, hf = lane >> 5;
    const long long L = a.seqlen;
    const long long q0 = (long long)qb * geo.qpw;
    const long long qw0 = q0 + 32 * (w / geo.hpw);                     // wave's first query
    const long long qrow = qw0 + r32;                                   // this lane's query
    const long long qlast = qw0 + 31 < L - 1 ? qw0 + 31 : L - 1;        // wave's last query

    // ---- the lane's query as 8 MFMA operands
    bf16x8 qop[D / 16];
    {
        const long long qr = qrow < L ? qrow : L - 1;
        load_q_operand(static_cast<const uint16_t *>(a.q) + ((b * L + qr) * a.q_heads + h) * (long long)D,
                       a.pos0 + qr, a.rope_dims, th, a.scale * 1.4426950408889634f, hf, qop);
    }

    f32x16 o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[c][v] = 0.f;
    float mrun = 0.f, lsum = 0.f;  // lane's reference maximum (log2 units) and sum
    f32x16 negm;                   // -mrun in every entry: where the score products start
#pragma unroll
    for (int v = 0; v < 16; ++v) negm[v] = 0.f;

    const long long kvh = (long long)b * L * a.kv_heads + g;  // row of token 0, K/V head g
    const uint16_t *kg = kr + kvh * D;
    const uint16_t *vg = static_cast<const uint16_t *>(a.v) + kvh * D;
    const int ts = a.kv_heads * D;                             // token stride (elements)
    const long long kend = q0 + geo.qpw < L ? q0 + geo.qpw : L; // keys [0, kend)
    const int nkb = (int)((kend + SKB - 1) / SKB);
    // staging: thread t holds block rows t/16 + (FNT/16) i, features
    // 8(t%16)..; rows past the end repeat the last key (masked later)
    constexpr int kSR = FNT / 16, kNR = SKB / kSR;  // rows per pass, passes
    const int srow = tid >> 4, scol = 8 * (tid & 15);
    u32x4 skr[kNR], svr[kNR];  // native vectors: arrays of uint4 (a union type) stayed in scratch
    // (indices fixed at compile time, so the staging stays in registers)
    // Byte offsets of the staged rows from a block's first row, unsigned 32-bit:
    // the block's base address is wave-uniform, so each load takes it from
    // scalar registers and adds its offset with no vector address arithmetic.
    const int nwhole = (int)(L / SKB);  // blocks [0, nwhole) lie inside the sequence
    uint32_t soff[kNR];
    static_for<kNR>([&](auto I) { soff[I] = (uint32_t)((srow + kSR * (int)I) * ts + scol) * 2u; });
    auto fa_load = [&](int kb) {
        const long long k0 = (long long)kb * SKB;
        const char *kb_ = reinterpret_cast<const char *>(kg + k0 * ts);
        const char *vb_ = reinterpret_cast<const char *>(vg + k0 * ts);
        if (kb < nwhole) {  // whole block (a 32-bit test, so it stays scalar)
            static_for<kNR>([&](auto I) {
                skr[I] = *reinterpret_cast<const u32x4 *>(kb_ + soff[I]);
                svr[I] = *reinterpret_cast<const u32x4 *>(vb_ + soff[I]);
            });
        } else {
            const int last = (int)(L - 1 - k0);
            static_for<kNR>([&](auto I) {
                const uint32_t o = (uint32_t)(min(srow + kSR * (int)I, last) * ts + scol) * 2u;
                skr[I] = *reinterpret_cast<const u32x4 *>(kb_ + o);
                svr[I] = *reinterpret_cast<const u32x4 *>(vb_ + o);
            });
        }
    };
    int wk[kNR], wv[kNR];  // tile offsets (elements) of the staged rows
    static_for<kNR>([&](auto I) {
        wk[I] = LK::off(srow + kSR * (int)I, scol);
        wv[I] = LV::off(srow + kSR * (int)I, scol);
    });
    const int kblast = (int)(qlast / SKB);  // the wave's last block with live keys
    if (nkb > 0) fa_load(0);
    // key block kb; MASKED: the block reaches the diagonal of some query of
    // the wave or the end of the sequence
    auto block = [&](int kb, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        // double-buffered tiles: buffer kb&1 was last read in block kb-2, which
        // every wave finished before the barrier of block kb-1
        __bf16 *Kb = Ks[kb & 1], *Vb = Vs[kb & 1];
        static_for<kNR>([&](auto I) {
            *reinterpret_cast<u32x4 *>(Kb + wk[I]) = skr[I];
            *reinterpret_cast<u32x4 *>(Vb + wv[I]) = svr[I];
        });
        if (kb + 1 < nkb) fa_load(kb + 1);
        __syncthreads();  // tiles visible
        if (kb > kblast) return;  // every key of this block is after the wave's queries
        const long long k0 = (long long)kb * SKB;

        // S^T blocks: keys k0 + 32kk.., this lane's query column; the two
        // halves interleave and each step's K operands load one step ahead
        // The products accumulate onto -m (negm), so sc holds s - m.
        f32x16 sc[2];
        {
            bf16x8 ka0 = ld_op<LK>(Kb, 0, 0, lane), ka1 = ld_op<LK>(Kb, 32, 0, lane);
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                bf16x8 kn0, kn1;
                if (ks + 1 < D / 16) {
                    kn0 = ld_op<LK>(Kb, 0, 16 * (ks + 1), lane);
                    kn1 = ld_op<LK>(Kb, 32, 16 * (ks + 1), lane);
                }
                sc[0] = mma(ka0, qop[ks], ks == 0 ? negm : sc[0]);
                sc[1] = mma(ka1, qop[ks], ks == 0 ? negm : sc[1]);
                ka0 = kn0;
                ka1 = kn1;
            }
        }
        // causal mask (and keys past the end); key 32kk + 8(v/4) + 4hf + v%4 of the block
        if constexpr (MASKED) {
            const int lim_q = (int)(qrow - k0);  // last key of this lane's query
            const int lim_l = (int)(L - 1 - k0 < SKB ? L - 1 - k0 : SKB);
            const int lim = lim_q < lim_l ? lim_q : lim_l;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (32 * kk + 8 * (v >> 2) + 4 * hf + (v & 3) > lim) sc[kk][v] = -__builtin_inff();
        }
        float mx = -__builtin_inff();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[kk][v]);
        // The reference maximum m (log2 units) is the first block's maximum
        // and afterwards moves only when a score exceeds it by more than
        // kStale: the probabilities stay below 2^kStale, and the rescale of O
        // and l (a wave-uniform branch) is rare after the first blocks. sc is
        // relative to m, so only a move of m subtracts anything from it. The
        // ballot sees every lane's own maximum; only a move needs the maximum
        // of the query's two lanes.
        if (kb == 0 || __builtin_amdgcn_ballot_w64(mx > kStale)) {
            // finite in block 0, where key 0 is live for every query; later, a
            // query with every key of the block masked has -inf and moves by 0
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float d = kb == 0 ? mx : fmaxf(mx, 0.f);  // the move of m
            if (kb != 0) {  // block 0 sets m: O and l are still zero
                const float alpha = __builtin_amdgcn_exp2f(-d);
#pragma unroll
                for (int c = 0; c < 4; ++c) o[c] *= alpha;
                lsum *= alpha;
            }
            mrun += d;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) sc[kk] -= d;
#pragma unroll
            for (int v = 0; v < 16; ++v) negm[v] = -mrun;
        }
        // P^T operands: step j holds keys 16j + 4hf + 0..3, 16j + 8 + 4hf + 0..3;
        // l sums the bf16 probabilities that enter the product
        bf16x8 pb[SKB / 16];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                pb[2 * kk + v / 8][v % 8] = static_cast<__bf16>(__builtin_amdgcn_exp2f(sc[kk][v]));
#pragma unroll
        for (int j = 0; j < SKB / 16; ++j)
#pragma unroll
            for (int e = 0; e < 8; e += 2)
                lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[j][e], pb[j][e + 1]}, kOnes2, lsum, false);
        {
            bf16x8 va[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) va[c] = ld_vt(Vb, 32 * c, 0, lane);
#pragma unroll
            for (int j = 0; j < SKB / 16; ++j) {
                bf16x8 vn[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (j + 1 < SKB / 16) vn[c] = ld_vt(Vb, 32 * c, 16 * (j + 1), lane);
                    o[c] = mma(va[c], pb[j], o[c]);
                }
#pragma unroll
                for (int c = 0; c < 4; ++c) va[c] = vn[c];
            }
        }
    };
    // Blocks that end at or before the first query of every wave and inside
    // the sequence take no mask (done as selects, the mask was a third of the
    // loop's vector instructions); the waves of a workgroup may differ in
    // their first query, so the split is at the smallest.
    const long long qmin = q0;  // first query of the workgroup
    int nfree = (int)((qmin + 1) / SKB);  // blocks [0, nfree): keys <= q0 for every query
    if ((long long)nfree * SKB > L) nfree = (int)(L / SKB);
    if (nfree > nkb) nfree = nkb;
    for (int kb = 0; kb < nfree; ++kb) block(kb, std::false_type{});
    for (int kb = nfree; kb < nkb; ++kb) block(kb, std::true_type{});

    // ---- normalise and store this lane's query row (value dims 32c + 8gv + 4hf..)
    lsum += __shfl_xor(lsum, 32);
    if (qrow < L) {
        const float inv = 1.f / lsum;
        OutT *og = static_cast<OutT *>(a.o) + ((b * L + qrow) * a.q_heads + h) * (long long)D;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int gv = 0; gv < 4; ++gv)
                put_out4<OutT>(og + 32 * c + 8 * gv + 4 * hf, o[c][4 * gv] * inv, o[c][4 * gv + 1] * inv,
                               o[c][4 * gv + 2] * inv, o[c][4 * gv + 3] * inv);
    }
}

// ---------------------------------------------------------------------------
// Decode

constexpr int DKB = 32;  // keys per decode block (one wave)
constexpr int kDecodeRec = 132;  // floats per partial record: O[128], m, l, 2 pad

// rope(k_new) into the key cache and v_new into the value cache at each
// sequence's position; 16 threads per (sequence, K/V head).
__global__ __launch_bounds__(SNT) void rope_append_kernel(SoftmaxDecodeArgs a) {
    __shared__ double th[kRopePairs];
    rope_table(th, a.rope_dims, a.log2_base, threadIdx.x, SNT);
    __syncthreads();
    const int row = blockIdx.x * (SNT / 16) + threadIdx.x / 16;
    if (row >= a.batch * a.kv_heads) return;
    const int b = row / a.kv_heads, g = row % a.kv_heads;
    const int n = a.lengths[b];
    if (n < 0 || n >= a.capacity) return;  // padding row
    const long long dst = (((long long)b * a.capacity + n) * a.kv_heads + g) * D;
    const int j = threadIdx.x % 16;
    *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.v_cache) + dst + 8 * j) =
        *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.v_new) + (long long)row * D + 8 * j);
    rope_row(static_cast<const uint16_t *>(a.k_new) + (long long)row * D,
             static_cast<uint16_t *>(a.k_cache) + dst, n, a.rope_dims, th, j);
}

// One wave per (sequence b, K/V head g, key split s): keys
// [s * chunk, min((s + 1) * chunk, n + 1)) with n = lengths[b], for the
// q_heads / kv_heads query heads of the group as MFMA columns. With one split
// the wave writes o; otherwise it writes its unnormalised partial (O, running
// max m in log2 units, sum l) for the combine kernel.
template <typename OutT>
__global__ __launch_bounds__(SNT) void fd_kernel(SoftmaxDecodeArgs a, int splits, long long chunk,
                                                 float *ws) {
    __shared__ __attribute__((aligned(16))) __bf16 Kw[4][DKB * SPT];
    __shared__ __attribute__((aligned(16))) __bf16 Vw[4][DKB * SPV];
    __shared__ double th[kRopePairs];  // filled before any wave can leave
    rope_table(th, a.rope_dims, a.log2_base, threadIdx.x, SNT);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const long long unit = (long long)blockIdx.x * 4 + w;
    if (unit >= (long long)a.batch * a.kv_heads * splits) return;
    const int s = (int)(unit % splits);
    const int bg = (int)(unit / splits);
    const int b = bg / a.kv_heads, g = bg % a.kv_heads;
    const int G = a.q_heads / a.kv_heads;
    const int r32 = lane & 31, hf = lane >> 5;
    const bool col = r32 < G;
    const int h = g * G + (col ? r32 : 0);
    const int n = a.lengths[b];
    const long long kbeg = (long long)s * chunk;
    if (n < 0 || n >= a.capacity) {  // padding row: zero output
        if (splits == 1 && col) {
            OutT *og = static_cast<OutT *>(a.o) + ((long long)b * a.q_heads + h) * D;
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int gv = 0; gv < 4; ++gv) put_out4<OutT>(og + 32 * c + 8 * gv + 4 * hf, 0.f, 0.f, 0.f, 0.f);
        }
        return;
    }
    if (kbeg > n) return;  // split past the sequence: the combine reads only live splits
    const long long kend = kbeg + chunk < (long long)n + 1 ? kbeg + chunk : (long long)n + 1;

    bf16x8 qop[D / 16];
    load_q_operand(static_cast<const uint16_t *>(a.q) + ((long long)b * a.q_heads + h) * D, n,
                   a.rope_dims, th, a.scale * 1.4426950408889634f, hf, qop);
    if (!col) {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) qop[ks][e] = static_cast<__bf16>(0.f);
    }

    const int ts = a.kv_heads * D;
    const long long base = ((long long)b * a.capacity * a.kv_heads + g) * D;  // token 0, head g
    const uint16_t *kc = static_cast<const uint16_t *>(a.k_cache) + base;
    const uint16_t *vc = static_cast<const uint16_t *>(a.v_cache) + base;
    __bf16 *Kt = Kw[w], *Vt = Vw[w];
    // staging: lane holds block rows (lane/16) + 4i, i = 0..7, features 8(lane%16)..
    const int srow = lane >> 4, scol = 8 * (lane & 15);
    uint4 sk[8], sv[8];
#define LT_FD_LOAD(K0)                                                                  \
    {                                                                                   \
        const long long k0_ = (K0);                                                     \
        const int last_ = kend - 1 - k0_ < DKB - 1 ? (int)(kend - 1 - k0_) : DKB - 1;   \
        const uint16_t *kb_ = kc + k0_ * ts, *vb_ = vc + k0_ * ts;                      \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                 \
            const int off_ = min(srow + 4 * i, last_) * ts + scol;                      \
            sk[i] = stream_load16(kb_ + off_);                                          \
            sv[i] = stream_load16(vb_ + off_);                                          \
        }                                                                               \
    }
    LT_FD_LOAD(kbeg)
    f32x16 o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[c][v] = 0.f;
    float mrun = -__builtin_inff(), lsum = 0.f;
    for (long long k0 = kbeg; k0 < kend; k0 += DKB) {
        // the wave's own tiles: DS instructions of one wave run in order, so
        // the previous block's reads are done before these writes land
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            *reinterpret_cast<uint4 *>(Kt + LK::off(srow + 4 * i, scol)) = sk[i];
            *reinterpret_cast<uint4 *>(Vt + LV::off(srow + 4 * i, scol)) = sv[i];
        }
        __builtin_amdgcn_wave_barrier();
        if (k0 + DKB < kend) LT_FD_LOAD(k0 + DKB)
        f32x16 sc;
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) sc = mma(ld_op<LK>(Kt, 0, 16 * ks, lane), qop[ks], sc);
        float mx = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            if (k0 + 8 * (v >> 2) + 4 * hf + (v & 3) >= kend) sc[v] = -__builtin_inff();
            mx = fmaxf(mx, sc[v]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(mrun, mx);  // finite: key k0 is live for every lane
        const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
        mrun = mnew;
        float ps = 0.f;
        bf16x8 pb[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float p = __builtin_amdgcn_exp2f(sc[v] - mnew);
            ps += p;
            pb[v / 8][v % 8] = static_cast<__bf16>(p);
        }
        lsum = lsum * alpha + ps;
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] *= alpha;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] = mma(ld_vt(Vt, 32 * c, 16 * j, lane), pb[j], o[c]);
        __builtin_amdgcn_wave_barrier();
    }
#undef LT_FD_LOAD
    lsum += __shfl_xor(lsum, 32);
    if (!col) return;
    if (splits == 1) {
        const float inv = 1.f / lsum;
        OutT *og = static_cast<OutT *>(a.o) + ((long long)b * a.q_heads + h) * D;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int gv = 0; gv < 4; ++gv)
                put_out4<OutT>(og + 32 * c + 8 * gv + 4 * hf, o[c][4 * gv] * inv, o[c][4 * gv + 1] * inv,
                               o[c][4 * gv + 2] * inv, o[c][4 * gv + 3] * inv);
    } else {
        float *rec = ws + (((long long)b * a.q_heads + h) * splits + s) * kDecodeRec;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int gv = 0; gv < 4; ++gv)
                *reinterpret_cast<float4 *>(rec + 32 * c + 8 * gv + 4 * hf) =
                    make_float4(o[c][4 * gv], o[c][4 * gv + 1], o[c][4 * gv + 2], o[c][4 * gv + 3]);
        if (hf == 0) *reinterpret_cast<float2 *>(rec + D) = make_float2(mrun, lsum);
    }
}

// Merges the live splits of each (sequence, query head): one thread per
// feature, o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <typename OutT>
__global__ __launch_bounds__(D) void fd_combine_kernel(SoftmaxDecodeArgs a, int splits, long long chunk,
                                                       const float *ws) {
    const int bh = blockIdx.x;
    const int b = bh / a.q_heads;
    const int t = threadIdx.x;
    OutT *og = static_cast<OutT *>(a.o) + (long long)bh * D + t;
    const int n = a.lengths[b];
    if (n < 0 || n >= a.capacity) {
        *og = static_cast<OutT>(0.f);
        return;
    }
    const int live = (int)(((long long)n + chunk) / chunk);  // splits holding keys 0..n
    const float *rec = ws + (long long)bh * splits * kDecodeRec;
    float M = -__builtin_inff();
    for (int s = 0; s < live; ++s) M = fmaxf(M, rec[(long long)s * kDecodeRec + D]);
    float l = 0.f, acc = 0.f;
    for (int s = 0; s < live; ++s) {
        const float *r = rec + (long long)s * kDecodeRec;
        const float e = __builtin_amdgcn_exp2f(r[D] - M);
        l += e * r[D + 1];
        acc += e * r[t];
    }
    *og = static_cast<OutT>(acc / l);
}

}  // namespace

hipError_t load_softmax_code() {
    hipFuncAttributes attr;
    return hipFuncGetAttributes(&attr, reinterpret_cast<const void *>(&fa_prefill_kernel<__bf16>));
}

hipError_t launch_softmax_prefill(const SoftmaxArgs &a, void *workspace, lt_dtype out_dtype,
                                  hipStream_t stream) {
    clear_pending_error();
    uint16_t *kr = static_cast<uint16_t *>(workspace);
    const long long rows = (long long)a.batch * a.seqlen * a.kv_heads;
    hipLaunchKernelGGL(rope_rows_kernel, dim3((unsigned)((rows + SNT / 16 - 1) / (SNT / 16))), dim3(SNT),
                       0, stream, a, kr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    FaGeom geo;
    const int G = a.q_heads / a.kv_heads;
    geo.hpw = std::gcd(G, FW);
    geo.qpw = 32 * FW / geo.hpw;
    geo.nqb = (int)((a.seqlen + geo.qpw - 1) / geo.qpw);
    geo.per_group = geo.nqb * (G / geo.hpw);
    geo.real = (long long)a.batch * a.kv_heads * geo.per_group;
    const dim3 grid((unsigned)((geo.real + 7) / 8 * 8));
    if (out_dtype == LT_F32)
        hipLaunchKernelGGL((fa_prefill_kernel<float>), grid, dim3(FNT), 0, stream, a, kr, geo);
    else
        hipLaunchKernelGGL((fa_prefill_kernel<__bf16>), grid, dim3(FNT), 0, stream, a, kr, geo);
    return hipGetLastError();
}

hipError_t launch_softmax_decode(const SoftmaxDecodeArgs &a, const SoftmaxDecodePlan &plan,
                                 float *workspace, lt_dtype out_dtype, hipStream_t stream) {
    clear_pending_error();
    const int rows = a.batch * a.kv_heads;
    hipLaunchKernelGGL(rope_append_kernel, dim3((rows + SNT / 16 - 1) / (SNT / 16)), dim3(SNT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long waves = (long long)rows * plan.splits;
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (out_dtype == LT_F32)
        hipLaunchKernelGGL((fd_kernel<float>), grid, dim3(SNT), 0, stream, a, plan.splits, plan.chunk, workspace);
    else
        hipLaunchKernelGGL((fd_kernel<__bf16>), grid, dim3(SNT), 0, stream, a, plan.splits, plan.chunk, workspace);
    e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
    const dim3 cgrid((unsigned)(a.batch * a.q_heads));
    if (out_dtype == LT_F32)
        hipLaunchKernelGGL((fd_combine_kernel<float>), cgrid, dim3(D), 0, stream, a, plan.splits, plan.chunk,
                           workspace);
    else
        hipLaunchKernelGGL((fd_combine_kernel<__bf16>), cgrid, dim3(D), 0, stream, a, plan.splits, plan.chunk,
                           workspace);
    return hipGetLastError();
}

}  // namespace lt
