// HIP kernels for gfx950 (MI355X): checkpoint + buffer decode step,
// conventional decode step, token-less flush and state reset.
//
// The method (blog "ReplaySSM: an SSM decoder that writes its state once
// every 16 tokens", sections "The identity" and "Output without a state";
// vLLM pull request "[Kernel] ReplaySSM: cache SSM inputs for faster Gated
// DeltaNet standard decode", reviewer comment on the output-only route):
// per head, with w records (lam_j, x_j, k_j) buffered since checkpoint C,
//   Mamba-2:  o = G (C q) + sum_j e_j (k_j . q) x_j + (k . q) v
//             G = exp(lam + sum_{l<w} lam_l), e_j = exp(lam + sum_{j<l<w} lam_l)
//   GDN:      S_{t-1} q = P (C q) + sum_j p_j (k_j . q) d_j, same with k,
//             P = exp(sum_{l<w} lam_l), p_j = exp(sum_{j<l<w} lam_l),
//             d = beta (v - alpha S_{t-1} k),  o = alpha S_{t-1} q + (k . q) d
// Decay weights are exponentials of suffix sums of log-decays (never a
// quotient of products), so every exponent is <= 0 and underflow gives 0.
//
// Work decomposition.  One workgroup owns one (row, head) tile for the whole
// step, so a flush may overwrite the checkpoint in place with no inter-
// workgroup hazard.  The d_v x d_k state tile is streamed once from HBM with
// 128-bit loads straight into registers: thread t of NT holds, for each of
// its NR passes, one 16-byte chunk of row (pass * RPP + t / LPR) at column
// chunk t % LPR.  Consecutive threads therefore read consecutive 16-byte
// chunks, and the LPR lanes sharing a state row form an aligned lane group
// inside one 64-wide wavefront.  Row sums (C q, C k) are finished with a
// halving exchange across the lane group, so NR row sums cost
// NR - 1 + log2(LPR) shuffles instead of NR log2(LPR).  The buffered records
// (at most L - 1 of them) are copied to LDS with 128-bit loads issued before
// the checkpoint loads, so their latency hides under the state stream.
// Everything after the row sums is row-local (one state row needs only its
// own sums and per-tile scalars), so a flush folds the records into the
// registers that already hold the tile and stores it once.
//
// Nothing here is bound by arithmetic: a non-flush step does about 2 FLOP per
// state byte-pair, so the kernels are designed around bytes in flight.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <vector>

#include "rs_internal.h"

namespace rs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- dtypes --
struct tF32 { using S = float; };
struct tF16 { using S = _Float16; };
struct tBF16 { using S = uint16_t; };
// OCP E4M3 codes: the read copy of a two-precision checkpoint only, each state
// row scaled by a power of two (kScaled).
struct tE4M3 { using S = uint8_t; };
template <class T> constexpr bool kScaled = false;
template <> constexpr bool kScaled<tE4M3> = true;

template <class T> __device__ __forceinline__ float to_f(typename T::S x);
template <> __device__ __forceinline__ float to_f<tF32>(float x) { return x; }
template <> __device__ __forceinline__ float to_f<tF16>(_Float16 x) { return (float)x; }
template <> __device__ __forceinline__ float to_f<tBF16>(uint16_t x) {
    return __uint_as_float((uint32_t)x << 16);
}

// Narrowing casts round to nearest even (the hardware's default mode for
// v_cvt_f16_f32); the round-toward-zero packed convert is never used.
template <class T> __device__ __forceinline__ typename T::S from_f(float x);
template <> __device__ __forceinline__ float from_f<tF32>(float x) { return x; }
template <> __device__ __forceinline__ _Float16 from_f<tF16>(float x) { return (_Float16)x; }
// bf16 keeps the top 16 bits of the float; round to nearest even on the
// discarded 16 (NaN stays a quiet NaN).
template <> __device__ __forceinline__ uint16_t from_f<tBF16>(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Load N consecutive elements (N * sizeof(S) bytes, naturally aligned to
// that size up to 16) and widen them to float.
template <class T, int N>
__device__ __forceinline__ void load_f(const typename T::S* __restrict__ p, float* out) {
    using S = typename T::S;
    constexpr int BYTES = N * (int)sizeof(S);
    S tmp[N];
    if constexpr (BYTES % 16 == 0) {
#pragma unroll
        for (int i = 0; i < BYTES / 16; ++i) {
            const u32x4 r = reinterpret_cast<const u32x4*>(p)[i];
            __builtin_memcpy(reinterpret_cast<char*>(tmp) + 16 * i, &r, 16);
        }
    } else if constexpr (BYTES == 8) {
        const u32x2 r = *reinterpret_cast<const u32x2*>(p);
        __builtin_memcpy(tmp, &r, 8);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) tmp[i] = p[i];
    }
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = to_f<T>(tmp[i]);
}

// Unpack one 16-byte chunk of state elements into floats.
template <class T>
__device__ __forceinline__ void unpack16(const u32x4 r, float* out) {
    using S = typename T::S;
    constexpr int N = 16 / sizeof(S);
    S tmp[N];
    __builtin_memcpy(tmp, &r, 16);
#pragma unroll
    for (int i = 0; i < N; ++i) out[i] = to_f<T>(tmp[i]);
}

template <class T>
__device__ __forceinline__ u32x4 pack16(const float* in) {
    using S = typename T::S;
    constexpr int N = 16 / sizeof(S);
    S tmp[N];
#pragma unroll
    for (int i = 0; i < N; ++i) tmp[i] = from_f<T>(in[i]);
    u32x4 r;
    __builtin_memcpy(&r, tmp, 16);
    return r;
}

// N elements of T held as N * sizeof(T) / 16 sixteen-byte chunks.  E4M3
// codes widen exactly (every code is an fp32 value), two per instruction;
// the row's scale is applied by the caller.
template <class T, int N>
__device__ __forceinline__ void unpack_n(const u32x4* in, float* out) {
    using S = typename T::S;
    if constexpr (kScaled<T>) {
        static_assert(N % 16 == 0, "whole chunks of codes");
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const int word = (int)in[i / 4][i % 4];
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
            out[4 * i] = lo[0];
            out[4 * i + 1] = lo[1];
            out[4 * i + 2] = hi[0];
            out[4 * i + 3] = hi[1];
        }
    } else {
        S tmp[N];
        __builtin_memcpy(tmp, in, sizeof(tmp));
#pragma unroll
        for (int i = 0; i < N; ++i) out[i] = to_f<T>(tmp[i]);
    }
}

template <class T, int N>
__device__ __forceinline__ void pack_n(const float* in, u32x4* out) {
    using S = typename T::S;
    S tmp[N];
#pragma unroll
    for (int i = 0; i < N; ++i) tmp[i] = from_f<T>(in[i]);
    __builtin_memcpy(out, tmp, sizeof(tmp));
}

template <int G>
__device__ __forceinline__ void group_max(float& x);  // below, with the other lane-group reductions

// One state row of E4M3 read copy (OCP 8-bit floating point specification:
// bias 7, largest finite 448).  The row's N * G values are spread over an
// aligned group of G lanes, N per lane.  Its scale is 2^e with e the smallest
// integer such that max|x| * 2^-e <= 448 (at least -100): with amax = f 2^E,
// f in [1, 2), that is e = E - 8, or E - 7 when f > 1.75, read off the bits
// of amax.  Scaling by 2^-e is exact (v_ldexp_f32), so the only rounding is
// the conversion to E4M3, to nearest even; no scaled value exceeds 448.
// Writes N codes to `codes` and returns the scale 2^e.
template <int N, int G>
__device__ __forceinline__ float encode_e4m3_row(const float* x, u32x4* codes) {
    static_assert(N % 16 == 0, "whole chunks of codes");
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < N; ++c) amax = fmaxf(amax, fabsf(x[c]));
    group_max<G>(amax);
    const uint32_t b = __float_as_uint(amax);
    int e = (int)((b >> 23) & 0xffu) - 127 - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
    e = max(e, -100);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(x[4 * i], -e),
                                                __builtin_amdgcn_ldexpf(x[4 * i + 1], -e), 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(x[4 * i + 2], -e),
                                            __builtin_amdgcn_ldexpf(x[4 * i + 3], -e), w, true);
        codes[i / 4][i % 4] = (uint32_t)w;
    }
    return __builtin_amdgcn_ldexpf(1.0f, e);
}

// Store one lane's share of a read-copy row (VEC values at `dst`); for a
// scaled format, lane 0 of the row's lane group also stores the row scale.
template <class TL, int VEC, int LPR>
__device__ __forceinline__ void store_read_row(const float* x, typename TL::S* dst, float* scale, int cc) {
    if constexpr (kScaled<TL>) {
        u32x4 codes[VEC / 16];
        const float sc = encode_e4m3_row<VEC, LPR>(x, codes);
#pragma unroll
        for (int i = 0; i < VEC / 16; ++i) __builtin_nontemporal_store(codes[i], reinterpret_cast<u32x4*>(dst) + i);
        if (cc == 0) *scale = sc;
    } else {
        u32x4 lo[VEC * sizeof(typename TL::S) / 16];
        pack_n<TL, VEC>(x, lo);
#pragma unroll
        for (int i = 0; i < (int)(VEC * sizeof(typename TL::S) / 16); ++i)
            __builtin_nontemporal_store(lo[i], reinterpret_cast<u32x4*>(dst) + i);
    }
}


// ------------------------------------------------------ stochastic rounding --
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC 2011): the published multipliers, Weyl key increments and
// round function; the key is advanced between rounds.
constexpr uint64_t kPhM0 = 0xD2E7470EE14C6C93ull, kPhM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhW0 = 0x9E3779B97F4A7C15ull, kPhW1 = 0xBB67AE8584CAA73Bull;

__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
#pragma unroll
    for (int rnd = 0; rnd < 10; ++rnd) {
        if (rnd) {
            k0 += kPhW0;
            k1 += kPhW1;
        }
        const uint64_t lo0 = kPhM0 * c[0], hi0 = __umul64hi(kPhM0, c[0]);
        const uint64_t lo1 = kPhM1 * c[2], hi1 = __umul64hi(kPhM1, c[2]);
        const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
    }
}

// fp32 -> fp16 bits with stochastic rounding by a 16-bit random word r:
// between the fp16 neighbours lo <= |x| < hi, take hi exactly when
// r < p 2^16, p = (|x| - lo) / (hi - lo).  For 2^-14 <= |x| < 65504 the
// fp32 value carries 13 bits m below the fp16 mantissa, p = m / 2^13, and
// r < 8 m is (r >> 3) < m: truncate, then add the carry (which may step into
// the next binade).  Below 2^-14 the neighbours are multiples of 2^-24:
// t = |x| 2^24 (exact), lo = floor(t), p = t - lo, and p 2^16 is exact.
// |x| >= 65504 and non-finite values round to nearest even.
__device__ __forceinline__ uint16_t sr_f16_bits(float x, uint32_t r) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t a = u & 0x7FFFFFFFu;
    const uint32_t sign = (u >> 16) & 0x8000u;
    if (a >= 0x38800000u && a < 0x477FE000u) {  // 2^-14 <= |x| < 65504
        const uint32_t up = (r >> 3) < (a & 0x1FFFu) ? 1u : 0u;
        return (uint16_t)((((a >> 13) - 0x1C000u) + up) | sign);
    }
    if (a >= 0x477FE000u) return __builtin_bit_cast(uint16_t, (_Float16)x);
    const float t = __uint_as_float(a) * 16777216.0f;
    const float lo = floorf(t);
    const uint32_t up = (float)r < __builtin_amdgcn_ldexpf(t - lo, 16) ? 1u : 0u;
    return (uint16_t)(((uint32_t)lo + up) | sign);
}

// Exchange with the adjacent lane (lane ^ 1), a DPP quad permutation.
__device__ __forceinline__ uint64_t xswap64(uint64_t v) {
    const int lo = __builtin_amdgcn_update_dpp((int)(uint32_t)v, (int)(uint32_t)v, 0xB1, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(uint32_t)(v >> 32), (int)(uint32_t)(v >> 32), 0xB1, 0xF, 0xF,
                                               false);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Random words for a lane's 8-element chunks (columns col .. col + 7, col a
// multiple of 8) of state rows row_first + r row_step, r < NR.  Element e of
// a (row, head) tile (row-major) uses 16-bit word e mod 16 of the
// Philox4x64-10 block for counter (sr_step, tile, e / 16, 0), the 64-bit
// outputs split least significant half-word first; a chunk is half a block,
// so w[r] = the two 64-bit outputs of its half.  The lane holding the other
// half of the same 16 columns is the adjacent one (lane ^ 1, column col ^ 8):
// with NR even each lane of the pair generates the block of one of two rows
// and hands the other half to its partner.  Every lane of the wave must
// execute this.
template <int NR>
__device__ __forceinline__ void sr_lane_words(const StepParams& p, int64_t tile, int row_first, int row_step,
                                              int dk, int col, uint64_t (&w)[NR][2]) {
    const bool odd = (col >> 3) & 1;
    const int64_t cblk = col >> 4;
    const int64_t bpr = dk / 16;  // blocks per state row
    if constexpr (NR % 2 == 0) {
#pragma unroll
        for (int r = 0; r < NR; r += 2) {
            const int row = row_first + (r + (odd ? 1 : 0)) * row_step;
            uint64_t c[4] = {p.sr_step, (uint64_t)tile, (uint64_t)(row * bpr + cblk), 0};
            philox4x64_10(c, p.sr_key0, p.sr_key1);
            const uint64_t k0 = odd ? c[2] : c[0], k1 = odd ? c[3] : c[1];
            const uint64_t g0 = xswap64(odd ? c[0] : c[2]), g1 = xswap64(odd ? c[1] : c[3]);
            w[r][0] = odd ? g0 : k0;
            w[r][1] = odd ? g1 : k1;
            w[r + 1][0] = odd ? k0 : g0;
            w[r + 1][1] = odd ? k1 : g1;
        }
    } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int row = row_first + r * row_step;
            uint64_t c[4] = {p.sr_step, (uint64_t)tile, (uint64_t)(row * bpr + cblk), 0};
            philox4x64_10(c, p.sr_key0, p.sr_key1);
            w[r][0] = odd ? c[2] : c[0];
            w[r][1] = odd ? c[3] : c[1];
        }
    }
}

// ------------------------------------------------------- lane-group sums --
// Partner exchange for the butterfly sums below, inside aligned groups of
// 2 * OFF lanes.  The sums only need, at level OFF, a pairing of each lane
// with one lane of the other half of its aligned group of 2 * OFF lanes (the
// lanes of a pair agree on every higher bit, so they hold the same partial
// sums, and each lane keeps the half selected by its own OFF bit).  That
// allows the cheap cross-lane forms of CDNA: DPP quad permutations for
// OFF = 1, 2 (lane ^ 1, lane ^ 2), DPP row half-mirror for OFF = 4 (lane i
// with 7 - i in its group of 8), DPP row mirror for OFF = 8 (i with 15 - i in
// its row of 16), and an LDS-free swizzle for OFF = 16 (lane ^ 16 in its
// group of 32); all are register moves, not LDS permutations.
template <int OFF>
__device__ __forceinline__ float xpartner(float x) {
    const int v = __float_as_int(x);
    int r;
    if constexpr (OFF == 1) r = __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false);        // quad_perm 1,0,3,2
    else if constexpr (OFF == 2) r = __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    else if constexpr (OFF == 4) r = __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    else if constexpr (OFF == 8) r = __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false);  // row_mirror
    else if constexpr (OFF == 16) r = __builtin_amdgcn_ds_swizzle(v, 0x401F);  // and 0x1f, xor 0x10
    else r = __float_as_int(__shfl_xor(x, OFF));
    return __int_as_float(r);
}

// Sum N per-lane values over an aligned group of lanes (offsets OFF, OFF/2,
// ..., 1; gl = lane index within the group).  While more than KEEP values are
// left, the lane whose OFF bit is set keeps the upper half of its values,
// its partner the lower half, and each adds the partner's copy of the half
// it keeps; once KEEP values are left, plain butterflies finish.  Afterwards
// the first xsum_left<N,G,KEEP>() entries of v hold complete sums of the
// contiguous original indices xsum_base<N,G,KEEP>(gl) + i, identical across
// the lanes that differ only in xsum_dup_mask<N,G,KEEP>() bits.
template <int N, int OFF, int KEEP = 1>
__device__ __forceinline__ void xsum(float* v, int gl) {
    if constexpr (OFF > 0) {
        if constexpr (N > KEEP) {
            const bool up = (gl & OFF) != 0;
#pragma unroll
            for (int i = 0; i < N / 2; ++i) {
                const float send = up ? v[i] : v[i + N / 2];
                const float keep = up ? v[i + N / 2] : v[i];
                v[i] = keep + xpartner<OFF>(send);
            }
            xsum<N / 2, OFF / 2, KEEP>(v, gl);
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) v[i] += xpartner<OFF>(v[i]);
            xsum<N, OFF / 2, KEEP>(v, gl);
        }
    }
}

template <int N, int G, int KEEP = 1>
constexpr int xsum_left() {
    int n = N;
    for (int o = G / 2; o > 0 && n > KEEP; o >>= 1) n /= 2;
    return n;
}

template <int N, int G, int KEEP = 1>
__device__ __forceinline__ int xsum_base(int gl) {
    int n = N, b = 0;
#pragma unroll
    for (int o = G / 2; o > 0 && n > KEEP; o >>= 1) {
        if (gl & o) b += n / 2;
        n /= 2;
    }
    return b;
}

template <int N, int G, int KEEP = 1>
constexpr int xsum_dup_mask() {
    int n = N, m = 0;
    for (int o = G / 2; o > 0; o >>= 1) {
        if (n > KEEP) n /= 2;
        else m |= o;
    }
    return m;
}

// Lane-bit mask that xpartner<OFF> flips: its pairs are lane ^ mask inside
// the group (row mirrors flip every lower bit too).
constexpr int flip_of(int off) { return off == 8 ? 15 : (off == 4 ? 7 : off); }
constexpr int parity(int x) { return __builtin_popcount(x) & 1; }

// Select-free first levels.  A lane whose N values are stored with their
// top index bits XOR-permuted can keep its lower half and send the upper half
// at each of the first PL levels, where xsum selects by the lane's own bit.
// Level l's permutation bit is m_l = parity(lane & A_l), with A_l chosen so
// that m_l differs between the lane and its partner at level l (they keep
// opposite halves) and is equal between the partners of every other level
// (earlier ones: the pair agrees on the order of what is left; later ones:
// the pair kept the same indices).  The pairings' lane masks are independent,
// so A_l is the dual basis vector, unique.  The kept original indices then
// have top bits m_0 m_1 ..., which xsum_perm_base accounts for; after the PL
// levels the remaining values are in natural order and xsum finishes.
template <int G, int L>
constexpr int xsum_perm_sel() {
    for (int a = 1; a < G; ++a) {
        bool ok = parity(flip_of((G / 2) >> L) & a) == 1;
        for (int k = 0; (G / 2) >> k > 0; ++k)
            if (k != L) ok = ok && parity(flip_of((G / 2) >> k) & a) == 0;
        if (ok) return a;
    }
    return 0;
}
template <int N, int OFF, int PL>
__device__ __forceinline__ void xsum_perm(float* v, int gl) {
    if constexpr (PL > 0 && OFF > 0) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) v[i] += xpartner<OFF>(v[i + N / 2]);
        xsum_perm<N / 2, OFF / 2, PL - 1>(v, gl);
    } else {
        xsum<N, OFF, 1>(v, gl);
    }
}

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// Levels of a group of G lanes that split an index of T values (a power of
// two, the top index bits first), and the XOR mask a lane applies to that
// index: bit (log2 T - 1 - l) is the lane's m_l.
template <int T, int G>
constexpr int xsum_perm_levels() {
    return ilog2(T) < ilog2(G) ? ilog2(T) : ilog2(G);
}
template <int T, int G>
__device__ __forceinline__ int xsum_perm_mask(int gl) {
    constexpr int LT = ilog2(T), PL = xsum_perm_levels<T, G>();
    static_assert(PL == 0 || xsum_perm_sel<G, 0>() != 0, "no select-free mask for this group");
    int m = 0;
    if constexpr (PL > 0) m |= parity(gl & xsum_perm_sel<G, 0>()) << (LT - 1);
    if constexpr (PL > 1) m |= parity(gl & xsum_perm_sel<G, 1>()) << (LT - 2);
    if constexpr (PL > 2) m |= parity(gl & xsum_perm_sel<G, 2>()) << (LT - 3);
    if constexpr (PL > 3) m |= parity(gl & xsum_perm_sel<G, 3>()) << (LT - 4);
    if constexpr (PL > 4) m |= parity(gl & xsum_perm_sel<G, 4>()) << (LT - 5);
    static_assert(PL <= 5, "levels");
    return m;
}
// First original index left in a lane after xsum_perm over N values whose
// top log2(T) bits are the permuted query index (mask xsum_perm_mask).
template <int N, int G, int T>
__device__ __forceinline__ int xsum_perm_base(int gl) {
    constexpr int PL = xsum_perm_levels<T, G>();
    constexpr int LT = ilog2(T);
    const int top = xsum_perm_mask<T, G>(gl) >> (LT - PL);  // the PL kept bits
    return top * (N >> PL) + xsum_base<(N >> PL), (G >> PL), 1>(gl);
}

// Plain butterfly sum of one value over the group; every lane gets the sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (G > 1) {
        x += xpartner<G / 2>(x);
        x = group_sum<G / 2>(x);
    }
    return x;
}

// Butterfly maximum over the group, in place; every lane gets the maximum.
template <int G>
__device__ __forceinline__ void group_max(float& x) {
    if constexpr (G > 1) {
        x = fmaxf(x, xpartner<G / 2>(x));
        group_max<G / 2>(x);
    }
}

// ------------------------------------------------------------ tile shape --
// A (row, head) tile of d_v x d_k state is covered by SPLIT workgroups, each
// owning DVW = d_v / SPLIT consecutive state rows (everything the step does is
// row-local except the record dot products, which each workgroup recomputes).
template <int DV, int DK, class TS, int SPLIT, int PER_ = 0>
struct Tile {
    using S = typename TS::S;
    static constexpr int DVW = DV / SPLIT;                     // state rows per workgroup
    static constexpr int VEC = 16 / (int)sizeof(S);           // state elements per 16 B
    static constexpr int LPR = DK / VEC;                       // lanes per state row
    static constexpr int LOADS = DVW * LPR;                    // 16-B chunks per workgroup
    // at least 4 chunks per thread, 2 for an E4M3 read copy (whose flush rows
    // hold 4 fp32 recurrence-copy chunks per code chunk), or PER_ if given
    static constexpr int PER = PER_ ? PER_ : (kScaled<TS> ? 2 : 4);
    static constexpr int NT = LOADS / PER >= 256 ? 256 : (LOADS / PER >= 128 ? 128 : 64);
    static constexpr int RPP = NT / LPR;                       // rows per pass
    static constexpr int NR = DVW / RPP;                       // passes per thread
    static_assert(DV % SPLIT == 0, "split");
    static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "lane group");
    static_assert(NT % LPR == 0 && DVW % RPP == 0 && NR >= 1, "tile split");
    static_assert((NR & (NR - 1)) == 0, "passes must be a power of two");
    static_assert(NT >= DVW && NT >= 64, "one thread per owned row, one full wave");
};

constexpr int kMamba2 = RS_MAMBA2;
constexpr int kGdn = RS_GDN;
// Whether a form's small writes are non-temporal (st_nt, below).
template <int FORM> constexpr bool kNtSmall = FORM == kMamba2;

struct TileIds {
    int row, head, part;
    int64_t tile;
};

// Grid: x = head * SPLIT + part, y = row.  The hardware hands workgroups to
// the 8 XCDs in turn by linear id (x + y * gridDim.x), and each XCD has its
// own L2.  Workgroups that read the same bytes form a unit of u = heads per
// key group * SPLIT consecutive tiles (the parts of a (row, head) tile share
// its records and token; the heads of a group share its key records, key and
// query), and a unit is mapped to one XCD: linear id i in a block of 8 u ids
// (b = i / 8u, r = i mod 8u) runs tile b 8u + (r mod 8) u + r / 8, so that
// the 8 units of a block go to the 8 XCDs and the members of a unit to the
// same one.  A last partial block keeps the identity.  Measured on MI355X
// (rocprofv3 FETCH_SIZE): with the identity, the 128-head Nemotron layer in
// 8 key groups fetched 7.5 % more than its algorithmic bytes at cursor 14
// (the group's keys read once per XCD rather than once per launch); mapped,
// its window average went from 199.7 to 189.5 us per launch, and Gated
// DeltaNet 128 x 128 with an fp32 state (two parts per tile) from 104.4 to
// 101.5 us.  With u = 1 (a key per head, whole tiles) the map is the identity.
constexpr int kXcds = 8;
template <int SPLIT>
__device__ __forceinline__ TileIds tile_ids(const StepParams& p) {
    TileIds t;
    const int u = p.heads_per_group * SPLIT;
    if (u == 1) {
        t.head = (int)blockIdx.x;
        t.part = 0;
        t.row = (int)blockIdx.y;
    } else {
        const int64_t W = gridDim.x;  // n_heads * SPLIT
        const int64_t i = (int64_t)blockIdx.y * W + blockIdx.x;
        const int64_t blk = (int64_t)kXcds * u;
        const int64_t full = (int64_t)gridDim.y * W / blk * blk;
        int64_t j = i;
        if (i < full) {
            const int64_t b = i / blk;
            const int r = (int)(i - b * blk);
            j = b * blk + (r % kXcds) * u + r / kXcds;
        }
        t.row = (int)(j / W);
        const int x = (int)(j - t.row * W);
        t.head = x / SPLIT;
        t.part = x - t.head * SPLIT;
    }
    t.tile = (int64_t)t.row * p.n_heads + t.head;
    return t;
}

// A row's flag byte, read as the 32-bit word that holds it (the array is
// 4-byte aligned, checked on the host): a uniform address, so this is a
// scalar load that issues together with the rest of the row metadata.  The
// word never leaves the 4-byte-aligned span of the flag itself.
__device__ __forceinline__ bool row_flag(const uint8_t* flags, int row) {
    const uint32_t word = reinterpret_cast<const uint32_t*>(flags)[row >> 2];
    return ((word >> (8 * (row & 3))) & 0xffu) != 0;
}

// A row's cursor word: the number of buffered records, and whether its
// checkpoint is zero and not to be read (RS_CURSOR_ZERO_CKPT: a row that
// joined and has not flushed yet).  A negative word stays negative, so the
// range checks still see it.
__device__ __forceinline__ int cursor_of(int word) { return word >= 0 ? (word & ~RS_CURSOR_ZERO_CKPT) : word; }
__device__ __forceinline__ bool zero_ckpt_of(int word) { return word >= 0 && (word & RS_CURSOR_ZERO_CKPT) != 0; }

// Counted once per (row, head) tile, by the workgroup owning its first rows.
__device__ __forceinline__ void count_error(const StepParams& p, const TileIds& id) {
    if (threadIdx.x == 0 && id.part == 0 && p.err) atomicAdd(p.err, 1);
}

// Streamed state and records are read or written once per step and are far
// larger than the caches, so they use non-temporal accesses (measured on
// MI355X: a 128-bit read stream moves from ~6.4 to ~7.2 TB/s, an in-place
// read-modify-write from ~5.3 to ~5.5-5.9 TB/s).
__device__ __forceinline__ u32x4 ld_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st_stream(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
// The small writes of a step (outputs, record appends, cursors): non-
// temporal for the Mamba-2 form, plain for Gated DeltaNet.  Measured on
// MI355X, batch 256: with plain stores the 20 MiB of outputs and record
// appends of a Nemotron-3-Super non-flush step cost about 16 us over the same
// step without them, with non-temporal stores about 5 us (window average
// 209.5 -> 199.3 us per launch; fp16 state 124.2 -> 121.6, E4M3 read copy
// 110.8 -> 108.8, conventional 365.9 -> 362.2); the Gated DeltaNet layers
// (32 heads, 128 x 128) were 1-2 % slower with them (fp32 state 105.0 ->
// 107.3 us, fp16 65.5 -> 66.3).
template <bool NT = true, class T>
__device__ __forceinline__ void st_nt(T* p, T v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Stores a lane's share of an fp16 state with stochastic rounding: HPC
// 8-element chunks per row, chunk h at column col0 + 8 LPR h (the lane order
// of a two-precision checkpoint; HPC = 1 for a single one), in rows
// row_first + r row_step (dst: the first chunk of the first of them, rows
// row_step d_k elements apart).  cf[r][8 h + i] is element i of chunk h.
template <int NR, int HPC, int LPR>
__device__ __forceinline__ void sr_store_rows(const float (&cf)[NR][8 * HPC], _Float16* dst, const StepParams& p,
                                              int64_t tile, int row_first, int row_step, int dk, int col0) {
    static_assert(HPC == 1 || LPR % 2 == 0, "the two halves of a block sit in adjacent lanes");
#pragma unroll
    for (int h = 0; h < HPC; ++h) {
        uint64_t w[NR][2];
        sr_lane_words<NR>(p, tile, row_first, row_step, dk, col0 + 8 * LPR * h, w);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            uint32_t o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint64_t wi = w[r][i >> 1];
                const int sh = 32 * (i & 1);
                const uint32_t b0 = sr_f16_bits(cf[r][8 * h + 2 * i], (uint32_t)(wi >> sh) & 0xFFFFu);
                const uint32_t b1 = sr_f16_bits(cf[r][8 * h + 2 * i + 1], (uint32_t)(wi >> (sh + 16)) & 0xFFFFu);
                o[i] = b0 | (b1 << 16);
            }
            st_stream(dst + (int64_t)r * row_step * dk + 8 * LPR * h, u32x4{o[0], o[1], o[2], o[3]});
        }
    }
}
// LDS carve-up shared by the step and flush kernels (DVW = rows owned).
template <class R>
struct Lds {
    R* k;         // [slots][DK]  buffered keys
    R* x;         // [slots][DVW] buffered values, owned rows
    float* e;     // [L]   per-record decay weight
    float* cq;    // [L]   k_j . q
    float* ck;    // [L]   k_j . k (Gated DeltaNet)
    float* v;     // [DVW] current v, owned rows
    float* u;     // [DVW] current corrected value d (Gated DeltaNet)
    float* sc;    // [4]   G, k . q
};

template <int DVW, int DK, class R>
__device__ __forceinline__ Lds<R> carve(char* smem, int slots, int L) {
    Lds<R> s;
    s.k = reinterpret_cast<R*>(smem);
    s.x = s.k + (int64_t)slots * DK;
    float* f = reinterpret_cast<float*>(s.x + (int64_t)slots * DVW);
    s.e = f;
    s.cq = s.e + L;
    s.ck = s.cq + L;
    s.v = s.ck + L;
    s.u = s.v + DVW;
    s.sc = s.u + DVW;
    return s;
}

template <int DVW, int DK, class R>
constexpr size_t lds_need(int slots, int L) {
    return (size_t)slots * (DK + DVW) * sizeof(R) + sizeof(float) * (3 * (size_t)L + 2 * DVW + 4);
}

// Copy records 0..w-1 into LDS in 16-byte chunks: keys (d_k each, contiguous
// in the buffer) then the owned DVW entries of each value record (stride d_v).
// issue() loads the first RC chunks per thread before the caller issues its
// checkpoint loads; commit() writes them to LDS afterwards and copies any
// remainder (only when w records exceed RC * NT chunks) directly.
template <int DV, int DVW, int DK, class R, int NT, int RC>
struct RecordCopy {
    static constexpr int KCH = DK * (int)sizeof(R) / 16;   // chunks per key record
    static constexpr int XCH = DVW * (int)sizeof(R) / 16;  // chunks per owned value record
    static constexpr int XE = 16 / (int)sizeof(R);         // elements per chunk
    static_assert(DK * sizeof(R) % 16 == 0 && DVW * sizeof(R) % 16 == 0, "record rows");
    u32x4 buf[RC];
    int nk, n;

    __device__ __forceinline__ const R* src(const R* rk, const R* rx, int i) const {
        if (i < nk) return rk + (int64_t)i * XE;
        const int t = i - nk, j = t / XCH;
        return rx + (int64_t)j * DV + (t - j * XCH) * XE;
    }
    // the same with no branch: w = 0 loads (and commit ignores) the first
    // chunk, so the ring must have a slot
    __device__ __forceinline__ void issue_always(const R* rk, const R* rx, int w) {
        nk = w * KCH;
        n = nk + w * XCH;
#pragma unroll
        for (int u = 0; u < RC; ++u) buf[u] = ld_stream(src(rk, rx, min(u * NT + (int)threadIdx.x, max(n - 1, 0))));
    }
    __device__ __forceinline__ void issue(const R* rk, const R* rx, int w) {
        nk = w * KCH;
        n = nk + w * XCH;
        if (n > 0) {  // uniform; loads clamped into range instead of predicated
#pragma unroll
            for (int u = 0; u < RC; ++u) buf[u] = ld_stream(src(rk, rx, min(u * NT + (int)threadIdx.x, n - 1)));
        }
    }
    // the same with no branch around the loads: with no records every lane
    // reads the 16 bytes at safe, which commit ignores
    __device__ __forceinline__ void issue_or(const R* rk, const R* rx, int w, const R* safe) {
        nk = w * KCH;
        n = nk + w * XCH;
#pragma unroll
        for (int u = 0; u < RC; ++u)
            buf[u] = ld_stream(n > 0 ? src(rk, rx, min(u * NT + (int)threadIdx.x, n - 1)) : safe);
    }
    // TAIL = false: the records fit the first RC * NT chunks (the caller
    // checked), so the remainder loop, whose loads would make the compiler
    // wait for every outstanding load, is left out.
    template <bool TAIL = true>
    __device__ __forceinline__ void commit(const R* rk, const R* rx, R* sk, R* sx) {
#pragma unroll
        for (int u = 0; u < RC; ++u) {
            const int i = u * NT + (int)threadIdx.x;
            if (i < n) {
                if (i < nk) reinterpret_cast<u32x4*>(sk)[i] = buf[u];
                else reinterpret_cast<u32x4*>(sx)[i - nk] = buf[u];
            }
        }
        if constexpr (TAIL)
        for (int i = RC * NT + (int)threadIdx.x; i < n; i += NT) {
            const u32x4 c = ld_stream(src(rk, rx, i));
            if (i < nk) reinterpret_cast<u32x4*>(sk)[i] = c;
            else reinterpret_cast<u32x4*>(sx)[i - nk] = c;
        }
    }
};

// Decay weights by a suffix scan over the lanes of wave 0, lane j holding
// lam_j for j < w (the buffer holds at most 63 records, so one wave covers
// it):  lane j < w writes e[j] = exp(base + sum_{j<l<w} lam_l), lane 0 writes
// sc[0] = G = exp(base + sum_{l<w} lam_l).  Every exponent is a sum of
// log-decays (<= 0), never a ratio of products.
__device__ __forceinline__ void decay_weights(float lam_j, float* e, float* sc, int w, float base) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        float s = lane < w ? lam_j : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {  // inclusive suffix sum over lanes >= lane
            const float t = __shfl_down(s, off);
            if (lane + off < 64) s += t;
        }
        float after = __shfl_down(s, 1);  // sum over lanes > lane
        if (lane == 63) after = 0.f;
        if (lane < w) e[lane] = expf(base + after);
        if (lane == 0) sc[0] = expf(base + s);
    }
}

// Cast N floats to the record type and store them (N * sizeof(R) bytes,
// aligned to that size up to 16).
template <class T, int N, bool NT = true>
__device__ __forceinline__ void store_f(typename T::S* __restrict__ p, const float* in) {
    using S = typename T::S;
    constexpr int BYTES = N * (int)sizeof(S);
    S tmp[N];
#pragma unroll
    for (int i = 0; i < N; ++i) tmp[i] = from_f<T>(in[i]);
    if constexpr (BYTES % 16 == 0) {
#pragma unroll
        for (int i = 0; i < BYTES / 16; ++i) {
            u32x4 r;
            __builtin_memcpy(&r, reinterpret_cast<const char*>(tmp) + 16 * i, 16);
            st_nt<NT>(reinterpret_cast<u32x4*>(p) + i, r);
        }
    } else if constexpr (BYTES == 8) {
        u32x2 r;
        __builtin_memcpy(&r, tmp, 8);
        st_nt<NT>(reinterpret_cast<u32x2*>(p), r);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) st_nt<NT>(p + i, tmp[i]);
    }
}

// ----------------------------------------------------- replay decode step --
// Order of work inside a workgroup:
//   1. row metadata (flag loaded first, consumed last);
//   2. small loads (token chunks, buffered decays and records), then the
//      checkpoint stream, so that waiting for the small loads never waits for
//      the stream;
//   3. records to LDS, barrier; decay weights and record dot products while
//      the checkpoint is still in flight; barrier;
//   4. per-lane partial sums of G (C q) plus this lane's share of the record
//      terms (lane c of a row's lane group takes records c, c + LPR, ...),
//      then one lane-group reduction that yields the output rows directly;
//   5. non-flush: append the record from registers; flush: fold and store.
//
// Two-precision checkpoint (TL != TS; blog "The precision argument,
// derived"): the block holds the recurrence copy (TS) and a read copy (TL).
// Non-flush rows stream only the read copy; a flush row loads the recurrence
// copy, folds in fp32 and stores both copies, each cast from the same
// unrounded values.  Threads are laid out by the read type: lane chunk cc of
// a row is one 16-byte read-copy chunk and HPC = sizeof(TS) / sizeof(TL)
// recurrence-copy chunks, which are chunks cc, cc + LPR, cc + 2 LPR, ... of
// the row, so that every load and store instruction of a wave covers
// contiguous memory (measured on MI355X: lanes that own consecutive chunks
// instead cut streaming writes from 5.6 to 2.3 TB/s at two chunks per lane
// and to 1.1 TB/s at four).  The read copy stores each row in the same lane
// order: its chunk cc holds the columns EPC (cc + LPR h) + i (h < HPC,
// i < EPC, EPC = recurrence-copy elements per 16 bytes).  q, k and buffered
// keys are read in that order too, so every dot product is unchanged.  With
// a single checkpoint HPC = 1 and the order is the natural one.
// RECON (Gated DeltaNet only): the state-reconstruction route, a separate
// instantiation so that the output-only route keeps its register budget.
// ROWS: kAllRows, or kNonFlushRows: an instantiation without the fold, which
// carries none of the flush path's registers and so keeps more waves in
// flight.  The caller's flush hint picks the kernels (RS_FLUSH_NONE: the
// second alone; RS_FLUSH_MIXED: the second over the rows that do not flush,
// then the first over those that do) and decides what a row that breaks it
// means: skipped, and counted as an error.
// kNonFlushRowsLong: the same without the fold, staging the records in 3
// chunks per thread instead of 2 (the persistent form copies them in one
// pass: rings of up to 32 records at 64 x 128 with fp16 records).
constexpr int kAllRows = 0, kNonFlushRows = 1, kNonFlushRowsLong = 2;
constexpr bool nonflush_rows(int rows) { return rows != kAllRows; }
constexpr int record_chunks(int rows) { return rows == kNonFlushRowsLong ? 3 : 2; }
constexpr int kMaxRecords = 63;  // a ring holds at most L - 1 <= 63 records
// The instantiation without the fold gives each thread 4 read-copy chunks
// (an E4M3 tile then takes 128 threads instead of 256): the fold's registers
// are gone, and twice the bytes per wave are in flight.
template <int DV, int DK, class TL, int SPLIT, int ROWS>
using StepTile = Tile<DV, DK, TL, SPLIT, nonflush_rows(ROWS) ? 4 : 0>;

// One non-flush tile's writes, held in LDS by a persistent workgroup until
// its tiles are done (see k_replay_step): the owned output rows, the record
// (key, owned value or corrected-value rows, log-decay) and where they go
// (work item = tile * SPLIT + part, block, cursor; cursor -1: nothing).
template <int DVW, int DK, class R>
struct Deferred {
    static constexpr int OUT = DVW * 4, KB = DK * (int)sizeof(R), XB = DVW * (int)sizeof(R);
    static constexpr int BYTES = OUT + KB + XB + 16;  // + work item, block, cursor, log-decay
    static_assert(OUT % 16 == 0 && KB % 16 == 0 && XB % 16 == 0, "16-byte pieces");
    float* out;
    R* k;
    R* x;
    int* meta;
    float* lam;
    __device__ __forceinline__ explicit Deferred(char* e)
        : out(reinterpret_cast<float*>(e)), k(reinterpret_cast<R*>(e + OUT)), x(reinterpret_cast<R*>(e + OUT + KB)),
          meta(reinterpret_cast<int*>(e + OUT + KB + XB)), lam(reinterpret_cast<float*>(e + OUT + KB + XB + 12)) {}
};

// N io elements of one lane, held as raw words from the load until they are
// used, so that a tile issued ahead of its arithmetic keeps its loads in
// flight.
template <class T, int N>
struct RawIo {
    using S = typename T::S;
    static constexpr int BYTES = N * (int)sizeof(S);
    static_assert(BYTES == 8 || BYTES % 16 == 0, "8 bytes or whole 16-byte chunks");
    uint32_t w[BYTES / 4];
    __device__ __forceinline__ void load(const S* __restrict__ p) {
        if constexpr (BYTES == 8) {
            const u32x2 r = *reinterpret_cast<const u32x2*>(p);
            w[0] = r[0];
            w[1] = r[1];
        } else {
#pragma unroll
            for (int i = 0; i < BYTES / 16; ++i) {
                const u32x4 r = reinterpret_cast<const u32x4*>(p)[i];
#pragma unroll
                for (int j = 0; j < 4; ++j) w[4 * i + j] = r[j];
            }
        }
    }
    __device__ __forceinline__ void to_float(float* out) const {
        S tmp[N];
        __builtin_memcpy(tmp, w, BYTES);
#pragma unroll
        for (int i = 0; i < N; ++i) out[i] = to_f<T>(tmp[i]);
    }
};

// Where one (row, head, part) tile's data lives.
template <int DV, int DK, class TS, class TR, class TI, class TL, int DVW>
struct TilePtrs {
    typename TS::S* ck;        // checkpoint (recurrence copy), owned rows
    typename TL::S* cl;        // read copy (two-precision checkpoint)
    float* cs;                 // read-copy row scales (scaled formats)
    typename TR::S* rx;        // value records, owned rows
    typename TR::S* rk;        // key records of the head's group
    float* rl;                 // log-decay records
    const typename TI::S* qp;  // this row's query, key and value tokens
    const typename TI::S* kp;
    const typename TI::S* vp;
    bool key_owner;            // the tile appends its group's key
    __device__ __forceinline__ TilePtrs(const StepParams& p, const TileIds& id, int blk) {
        using S = typename TS::S;
        using RL = typename TL::S;
        using R = typename TR::S;
        using I = typename TI::S;
        const int row0 = id.part * DVW;
        char* base = p.pool + (int64_t)blk * p.block_bytes;
        ck = reinterpret_cast<S*>(base + p.ckpt_off) + (int64_t)id.head * (DV * DK) + (int64_t)row0 * DK;
        cl = reinterpret_cast<RL*>(base + p.ckpt_lo_off) + (int64_t)id.head * (DV * DK) + (int64_t)row0 * DK;
        cs = reinterpret_cast<float*>(base + p.ckpt_sc_off) + id.head * DV + row0;
        rx = reinterpret_cast<R*>(base + p.recx_off) + (int64_t)id.head * p.slots * DV + row0;
        // keys and queries per group of heads_per_group heads (1: per head)
        const int grp = id.head / p.heads_per_group;
        key_owner = id.head == grp * p.heads_per_group;
        // (the step kernels run standard layers only, where key_slots == slots)
        rk = reinterpret_cast<R*>(base + p.reck_off) + (int64_t)grp * p.slots * DK;
        rl = reinterpret_cast<float*>(base + p.reclam_off) + (int64_t)id.head * p.slots;
        qp = static_cast<const I*>(p.q) + id.row * p.qs_r + grp * p.qs_h;
        kp = static_cast<const I*>(p.k) + id.row * p.ks_r + grp * p.ks_h;
        vp = static_cast<const I*>(p.v) + id.row * p.vs_r + id.head * p.vs_h + row0;
    }
};

// A tile's loads (tile_issue_small, tile_issue_stream) and whether it runs; tile_finish
// does its arithmetic and stores.  The two halves let a persistent
// workgroup issue the next tile's loads before it computes the current one.
template <int FORM, int DV, int DK, class TS, class TR, class TI, int SPLIT, class TL, int ROWS>
struct TileIn {
    using T = StepTile<DV, DK, TL, SPLIT, ROWS>;
    static constexpr int VEC = T::VEC, NR = T::NR, NT = T::NT, DVW = T::DVW;
    static constexpr int HPC = VEC * (int)sizeof(typename TS::S) / 16;  // recurrence-copy chunks per lane chunk
    static constexpr int EPC = VEC / HPC;                               // elements per recurrence-copy chunk
    TileIds id;
    int blk, w;
    bool run, fl;  // the tile is computed here; it flushes
    bool zc;       // the row's checkpoint is zero (RS_CURSOR_ZERO_CKPT): not read
    RawIo<TI, EPC> qr[HPC], kr[HPC];
    typename TI::S vr;
    float lam, lam_j;
    float beta;  // Gated DeltaNet
    RecordCopy<DV, DVW, DK, typename TR::S, NT, record_chunks(ROWS)> rec;
    float rsc[NR];  // scales of the owned read-copy rows (scaled formats)
    u32x4 cb[NR * HPC];
};

// Whether a tile runs in this launch, and whether it flushes, from its row's
// metadata; a skipped tile is counted as an error where the flush hint's
// rules say so.  ERR_LDS (persistent workgroups, one item per thread while
// they stage their items): counted in LDS, so that no global write is
// pending in the loop that issues ahead (the compiler then waits for every
// outstanding load at once).
template <int ROWS, bool ERR_LDS = false>
__device__ __forceinline__ bool tile_runs(const StepParams& p, const TileIds& id, int blk, int w, bool flag, bool& fl,
                                          int* err_lds = nullptr) {
    fl = false;
    if (blk < 0) return false;  // padding
    auto error = [&]() {
        if constexpr (ERR_LDS) {
            if (id.part == 0) atomicAdd(err_lds, 1);
        } else {
            count_error(p, id);
        }
    };
    if (blk >= p.n_blocks || w < 0 || w > p.slots) {
        // a pair of launches counts a bad tile once, in the first
        if (!(ROWS == kAllRows && p.flush_hint == RS_FLUSH_MIXED)) error();
        return false;
    }
    const bool fl_row = (w == p.slots) || flag;
    if constexpr (nonflush_rows(ROWS)) {
        if (fl_row) {
            if (p.flush_hint == RS_FLUSH_NONE) error();  // the hint was wrong
            return false;
        }
        return true;
    } else {
        if (!fl_row && (p.flush_hint == RS_FLUSH_ALL || p.flush_hint == RS_FLUSH_MIXED)) {
            if (p.flush_hint == RS_FLUSH_ALL) error();
            return false;
        }
        fl = fl_row;
        return true;
    }
}

// The small loads of a tile that runs (tokens, buffered decays and records;
// the checkpoint stream is tile_issue_stream's), issued before the stream so
// that waiting for them never waits for the stream.  UNCOND (tiles that do
// not flush, so the ring has a slot 0): no branch around any load, a ring
// with no records yet reading slot 0 and ignoring it, so that a loop that
// issues ahead has none either.
template <int FORM, int DV, int DK, class TS, class TR, class TI, int SPLIT, class TL, int ROWS, bool UNCOND = false>
__device__ __forceinline__ void tile_issue_small(const StepParams& p, const TileIds id, int blk, int w, bool fl, bool zc,
                                                 TileIn<FORM, DV, DK, TS, TR, TI, SPLIT, TL, ROWS>& in) {
    using In = TileIn<FORM, DV, DK, TS, TR, TI, SPLIT, TL, ROWS>;
    using T = typename In::T;
    constexpr int LPR = T::LPR, RPP = T::RPP, NR = T::NR, DVW = T::DVW;
    constexpr bool SC = kScaled<TL>;
    constexpr int HPC = In::HPC, EPC = In::EPC;
    static_assert(!UNCOND || nonflush_rows(ROWS), "unconditional loads: non-flush tiles only");

    in.id = id;
    in.blk = blk;
    in.w = w;
    in.run = true;
    in.fl = fl;
    in.zc = zc;
    const int tid = threadIdx.x;
    const int cc = tid % LPR;  // column chunk
    const int rg = tid / LPR;  // row within a pass
    const TilePtrs<DV, DK, TS, TR, TI, TL, DVW> P(p, id, blk);
    in.lam = p.lam[id.tile];
    if constexpr (FORM == kGdn) in.beta = p.beta[id.tile];
    // column of element h * EPC + i of this lane's share of a row
    const int col0 = EPC * cc;
#pragma unroll
    for (int h = 0; h < HPC; ++h) {
        in.qr[h].load(P.qp + col0 + EPC * LPR * h);
        in.kr[h].load(P.kp + col0 + EPC * LPR * h);
    }
    in.vr = P.vp[min(tid, DVW - 1)];
    if constexpr (UNCOND) {
        in.lam_j = P.rl[min(tid, max(w - 1, 0))];
        in.rec.issue_always(P.rk, P.rx, w);
    } else {
        // no branch around these loads either: an empty ring reads a valid
        // address and ignores the value (see tile_issue_stream)
        const float* lp = w > 0 ? P.rl + min(tid, w - 1) : p.lam + id.tile;
        const float lj = *lp;
        in.lam_j = w > 0 ? lj : 0.f;
        in.rec.issue_or(P.rk, P.rx, w, reinterpret_cast<const typename TR::S*>(P.ck));
    }
    if constexpr (SC) {
        if (!fl) {
#pragma unroll
            for (int r = 0; r < NR; ++r) in.rsc[r] = P.cs[r * RPP + rg];
        }
    }
}

// The checkpoint stream of a tile whose small loads tile_issue_small issued.
// always: issue the loads even for a zero checkpoint (its values are then
// replaced by zeros in tile_finish), so that a loop issuing ahead has no
// branch around them; otherwise a zero checkpoint's loads all read the
// tile's first 16 bytes (one checkpoint) or are skipped (two copies).
template <int FORM, int DV, int DK, class TS, class TR, class TI, int SPLIT, class TL, int ROWS>
__device__ __forceinline__ void tile_issue_stream(const StepParams& p,
                                                  TileIn<FORM, DV, DK, TS, TR, TI, SPLIT, TL, ROWS>& in,
                                                  bool always = false) {
    using In = TileIn<FORM, DV, DK, TS, TR, TI, SPLIT, TL, ROWS>;
    using T = typename In::T;
    using S = typename TS::S;
    constexpr int VEC = T::VEC, LPR = T::LPR, RPP = T::RPP, NR = T::NR, DVW = T::DVW;
    constexpr bool TWO = !std::is_same<TS, TL>::value;
    constexpr int HPC = In::HPC, EPC = In::EPC;
    const bool fl = in.fl;
    const int tid = threadIdx.x;
    const int cc = tid % LPR;
    const int rg = tid / LPR;
    const int col0 = EPC * cc;
    const TilePtrs<DV, DK, TS, TR, TI, TL, DVW> P(p, in.id, in.blk);
    if constexpr (TWO)
        if (in.zc && !always) return;
    // A single checkpoint's stream is issued even for a zero checkpoint, every
    // lane then reading the tile's first 16 bytes (one cache line, ignored):
    // with a branch around these loads the compiler makes the record copy
    // wait for the whole stream (its wait counts cover both paths).
    const bool skip = !TWO && in.zc && !always;
    if (!TWO || fl) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const S* rowp = P.ck + (int64_t)(r * RPP + rg) * DK + col0;
#pragma unroll
            for (int h = 0; h < HPC; ++h) in.cb[r * HPC + h] = ld_stream(skip ? P.ck : rowp + EPC * LPR * h);
        }
    } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) in.cb[r * HPC] = ld_stream(P.cl + (int64_t)(r * RPP + rg) * DK + cc * VEC);
    }
}

template <int FORM, int DV, int DK, class TS, class TR, class TI, int SPLIT, class TL, bool RECON, int ROWS,
          bool DEFER>
__device__ __forceinline__ void tile_finish(const StepParams& p,
                                            const TileIn<FORM, DV, DK, TS, TR, TI, SPLIT, TL, ROWS>& in, char* smem,
                                            char* dslot) {
    using In = TileIn<FORM, DV, DK, TS, TR, TI, SPLIT, TL, ROWS>;
    using T = typename In::T;
    using S = typename TS::S;
    using R = typename TR::S;
    constexpr int VEC = T::VEC, LPR = T::LPR, RPP = T::RPP, NR = T::NR, DVW = T::DVW;
    constexpr int KEEP = FORM == kGdn ? 2 : 1;  // Gated DeltaNet keeps (C q, C k) of a row together
    constexpr int NV = KEEP * NR;
    constexpr bool TWO = !std::is_same<TS, TL>::value;
    constexpr bool SC = kScaled<TL>;                // read copy with per-row scales
    constexpr int HPC = In::HPC, EPC = In::EPC;

    static_assert(!DEFER || nonflush_rows(ROWS), "deferred writes: non-flush rows only");
    using D = Deferred<DVW, DK, R>;
    D df(dslot);
    if (!in.run) {
        if constexpr (DEFER)
            if (threadIdx.x == 0) df.meta[2] = -1;  // nothing to write
        return;
    }
    const TileIds id = in.id;
    const int blk = in.blk, w = in.w;
    const bool fl = in.fl;
    if constexpr (DEFER) {
        if (threadIdx.x == 0) {
            df.meta[0] = (int)id.tile * SPLIT + id.part;
            df.meta[1] = blk;
            df.meta[2] = w | (in.zc ? RS_CURSOR_ZERO_CKPT : 0);
        }
    }

    const int tid = threadIdx.x;
    const int cc = tid % LPR;  // column chunk
    const int rg = tid / LPR;  // row within a pass
    const int row0 = id.part * DVW;
    const TilePtrs<DV, DK, TS, TR, TI, TL, DVW> P(p, id, blk);
    S* ck = P.ck;
    typename TL::S* cl = P.cl;
    float* cs = P.cs;
    R* rx = P.rx;
    R* rk = P.rk;
    float* rl = P.rl;
    const bool key_owner = P.key_owner;
    const float lam = in.lam;

    const Lds<R> s = carve<DVW, DK, R>(smem, p.slots, p.L);

    const int col0 = EPC * cc;
    auto col = [col0](int h) { return col0 + EPC * LPR * h; };
    float qv[VEC], kv[VEC];
#pragma unroll
    for (int h = 0; h < HPC; ++h) {
        in.qr[h].to_float(qv + h * EPC);
        in.kr[h].to_float(kv + h * EPC);
    }
    const float vi = to_f<TI>(in.vr);
    // a non-flush row's record: log-decay, key (one per group), value
    // (Mamba-2; Gated DeltaNet stores its corrected value with the output)
    auto append_record = [&](int slot) {
        if (id.part == 0) {
            if (tid == 0) {
                if constexpr (DEFER) *df.lam = lam;
                else st_nt<kNtSmall<FORM>>(rl + slot, lam);
            }
            if (rg == 0 && key_owner) {
                R* kd = DEFER ? df.k + col0 : rk + (int64_t)slot * DK + col0;
#pragma unroll
                for (int h = 0; h < HPC; ++h) store_f<TR, EPC, kNtSmall<FORM>>(kd + EPC * LPR * h, kv + h * EPC);
            }
        }
        if constexpr (FORM == kMamba2) {
            if (tid < DVW) {
                if constexpr (DEFER) df.x[tid] = from_f<TR>(vi);
                else st_nt<kNtSmall<FORM>>(rx + (int64_t)slot * DV + tid, from_f<TR>(vi));
            }
        }
    };
    const float lam_j = in.lam_j;
    auto rec = in.rec;
    float rsc[NR];
    u32x4 cb[NR * HPC];
#pragma unroll
    for (int r = 0; r < NR; ++r) rsc[r] = in.rsc[r];
#pragma unroll
    for (int i = 0; i < NR * HPC; ++i) cb[i] = in.cb[i];
    // A zero checkpoint: zero bits are +0 in every state and read format.  The
    // one-workgroup kernel clears its registers after the record work below,
    // since overwriting them here would wait for the checkpoint stream.
    if (DEFER && in.zc) {
#pragma unroll
        for (int r = 0; r < NR; ++r) rsc[r] = 1.0f;
#pragma unroll
        for (int i = 0; i < NR * HPC; ++i) cb[i] = u32x4{0u, 0u, 0u, 0u};
    }

    if (tid < DVW) s.v[tid] = vi;
    rec.template commit<!DEFER>(rk, rx, s.k, s.x);
    // The kernel without the fold appends the record (slot w, which this
    // step does not read) and takes this lane's share of k . q now, so that
    // k is not held through the checkpoint products.
    float kq_lane = 0.f;
    if constexpr (nonflush_rows(ROWS)) {
#pragma unroll
        for (int c = 0; c < VEC; ++c) kq_lane += kv[c] * qv[c];
        append_record(w);
    }
    __syncthreads();

    decay_weights(lam_j, s.e, s.sc, w, FORM == kMamba2 ? lam : 0.0f);

    // Gated DeltaNet, state-reconstruction route: S_{t-1} is rebuilt in
    // registers below, so no record dot products are needed.
    constexpr bool recon = FORM == kGdn && RECON;
    const int wd = recon ? 0 : w;  // records whose dot products are taken

    // Record dot products: lane group rg takes records rg, rg + RPP, ...;
    // index wd stands for the current token (k . q).
    const int rounds = (wd + RPP) / RPP;
    for (int it = 0; it < rounds; ++it) {
        const int j = it * RPP + rg;
        float kj[VEC];
        if (j < wd) {
#pragma unroll
            for (int h = 0; h < HPC; ++h) load_f<TR, EPC>(s.k + (int64_t)j * DK + col(h), kj + h * EPC);
        } else if constexpr (!nonflush_rows(ROWS)) {
#pragma unroll
            for (int c = 0; c < VEC; ++c) kj[c] = kv[c];
        }
        float pq = 0.f, pk = 0.f;
        if (nonflush_rows(ROWS) && j >= wd) {
            pq = kq_lane;
        } else {
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                pq += kj[c] * qv[c];
                if constexpr (FORM == kGdn) pk += kj[c] * kv[c];
            }
        }
        pq = group_sum<LPR>(pq);
        if constexpr (FORM == kGdn) pk = group_sum<LPR>(pk);
        if (cc == 0 && j <= wd) {
            if (j < wd) {
                s.cq[j] = pq;
                if constexpr (FORM == kGdn) s.ck[j] = pk;
            } else {
                s.sc[1] = pq;
            }
        }
    }
    __syncthreads();

    if (!DEFER && in.zc) {
#pragma unroll
        for (int r = 0; r < NR; ++r) rsc[r] = 1.0f;
#pragma unroll
        for (int i = 0; i < NR * HPC; ++i) cb[i] = u32x4{0u, 0u, 0u, 0u};
    }
    const float G = s.sc[0];
    const float kq = s.sc[1];
    float cf[NR][VEC];
    if (!TWO || fl) {
#pragma unroll
        for (int r = 0; r < NR; ++r) unpack_n<TS, VEC>(&cb[r * HPC], cf[r]);
    } else if constexpr (!(nonflush_rows(ROWS) && SC)) {
#pragma unroll
        for (int r = 0; r < NR; ++r) unpack_n<TL, VEC>(&cb[r * HPC], cf[r]);
    }
    if constexpr (FORM == kGdn) {
        if constexpr (recon) {  // S_{t-1} = G C + sum_j e_j d_j k_j^T
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int c = 0; c < VEC; ++c) cf[r][c] *= G;
            for (int j = 0; j < w; ++j) {
                float kj[VEC];
                load_f<TR, VEC>(s.k + (int64_t)j * DK + col0, kj);
                const float ej = s.e[j];
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const float f = ej * to_f<TR>(s.x[(int64_t)j * DVW + r * RPP + rg]);
#pragma unroll
                    for (int c = 0; c < VEC; ++c) cf[r][c] += f * kj[c];
                }
            }
        }
    }
    const float gs = recon ? 1.0f : G;  // the checkpoint's weight in the products below
    float acc[NV];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        float a = 0.f, b = 0.f;
        if constexpr (nonflush_rows(ROWS) && SC) {
            // codes widened four at a time straight into the product, so
            // that the tile is never held as floats
#pragma unroll
            for (int i = 0; i < VEC / 4; ++i) {
                const int word = (int)cb[r * HPC + i / 4][i % 4];
                const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
                const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
                a += lo[0] * qv[4 * i] + lo[1] * qv[4 * i + 1] + hi[0] * qv[4 * i + 2] + hi[1] * qv[4 * i + 3];
            }
        } else {
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                a += cf[r][c] * qv[c];
                if constexpr (FORM == kGdn) b += cf[r][c] * kv[c];
            }
        }
        if constexpr (FORM == kMamba2) {
            if constexpr (SC) a = fl ? a : rsc[r] * a;
            acc[r] = G * a;
        } else {
            acc[2 * r] = gs * a;
            acc[2 * r + 1] = gs * b;
        }
    }
    auto record_terms = [&](int j) {
        const float wq = s.e[j] * s.cq[j];
        const float wk = FORM == kGdn ? s.e[j] * s.ck[j] : 0.f;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const float xj = to_f<TR>(s.x[(int64_t)j * DVW + r * RPP + rg]);
            if constexpr (FORM == kMamba2) {
                acc[r] += wq * xj;
            } else {
                acc[2 * r] += wq * xj;
                acc[2 * r + 1] += wk * xj;
            }
        }
    };
    if constexpr (DEFER) {
        // (unrolled to its bound, at most 63 records: a per-lane loop here
        // makes the compiler wait for the prefetched loads)
#pragma unroll
        for (int it = 0; it < (kMaxRecords + LPR - 1) / LPR; ++it)
            if (cc + it * LPR < wd) record_terms(cc + it * LPR);
    } else {
        for (int j = cc; j < wd; j += LPR) record_terms(j);
    }
    if constexpr (FORM == kMamba2) {
        if (cc == LPR - 1) {
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[r] += kq * s.v[r * RPP + rg];
        }
    }
    xsum<NV, LPR / 2, KEEP>(acc, cc);

    if constexpr (!DEFER)  // (deferred: stored with the item's other writes)
        if (p.next_wp && id.head == 0 && id.part == 0 && tid == 0)
            st_nt<kNtSmall<FORM>>(p.next_wp + id.row, fl ? 0 : (w + 1) | (in.zc ? RS_CURSOR_ZERO_CKPT : 0));
    const float alpha = expf(lam);  // Gated DeltaNet only
    float* o = DEFER ? df.out : p.out + id.tile * DV + row0;
    // One-workgroup tiles stage the output rows (and Gated DeltaNet's
    // corrected values) in LDS and store them below in whole 16-byte chunks:
    // the lanes holding the reduced rows cover rows RPP apart, and storing
    // from them scatters small pieces into the checkpoint read stream.
    // Mamba-2 stages its outputs in u (unused by that form); Gated DeltaNet
    // stages them in v (a row's v is read just before, by the same lane) and
    // its corrected values in u, where the flush fold reads them.
    constexpr bool STAGE = !DEFER && DVW % 4 == 0 && (DVW * (int)sizeof(R)) % 16 == 0;
    float* so = FORM == kMamba2 ? s.u : s.v;
    {
        constexpr int left = xsum_left<NV, LPR, KEEP>();
        const int b0 = xsum_base<NV, LPR, KEEP>(cc);
        if ((cc & xsum_dup_mask<NV, LPR, KEEP>()) == 0) {
            if constexpr (FORM == kMamba2) {
#pragma unroll
                for (int i = 0; i < left; ++i) {
                    if constexpr (STAGE) so[(b0 + i) * RPP + rg] = acc[i];
                    else st_nt(o + (b0 + i) * RPP + rg, acc[i]);
                }
            } else {
                const float bt = in.beta;
#pragma unroll
                for (int i = 0; i < left; i += 2) {
                    const int row = ((b0 + i) / 2) * RPP + rg;
                    const float d = bt * (s.v[row] - alpha * acc[i + 1]);
                    if constexpr (STAGE) {
                        so[row] = alpha * acc[i] + kq * d;
                        s.u[row] = d;
                    } else {
                        st_nt<kNtSmall<FORM>>(o + row, alpha * acc[i] + kq * d);
                        if (fl) s.u[row] = d;
                        else if constexpr (DEFER) df.x[row] = from_f<TR>(d);
                        else st_nt<kNtSmall<FORM>>(rx + (int64_t)w * DV + row, from_f<TR>(d));
                    }
                }
            }
        }
    }
    if constexpr (STAGE) {
        __syncthreads();
        constexpr int OC = DVW / 4;                     // output chunks
        constexpr int XE = 16 / (int)sizeof(R);         // record elements per chunk
        constexpr int XC = FORM == kGdn ? DVW / XE : 0;  // corrected-value chunks
        static_assert(OC + XC <= T::NT, "one chunk per thread");
        if (tid < OC) {
            st_nt<kNtSmall<FORM>>(reinterpret_cast<u32x4*>(o) + tid,
                                  u32x4{__float_as_uint(so[4 * tid]), __float_as_uint(so[4 * tid + 1]),
                                        __float_as_uint(so[4 * tid + 2]), __float_as_uint(so[4 * tid + 3])});
        } else if (FORM == kGdn && !fl && tid < OC + XC) {
            const int c = tid - OC;
            float dv[XE];
#pragma unroll
            for (int e = 0; e < XE; ++e) dv[e] = s.u[c * XE + e];
            store_f<TR, XE, kNtSmall<FORM>>(rx + (int64_t)w * DV + c * XE, dv);
        }
    }

    if (!fl) {  // uniform across the workgroup
        if constexpr (!nonflush_rows(ROWS)) append_record(w);  // (else appended above)
        return;
    }

    // Flush: fold records and the current token into the registers holding
    // the owned rows, store once.
    //   Mamba-2:  C' = G C + sum_j e_j x_j k_j^T + v k^T
    //   GDN:      C' = alpha P C + sum_j alpha p_j d_j k_j^T + d k^T
    if constexpr (FORM == kGdn && !STAGE) __syncthreads();  // d in LDS (staged: stored above)
    // (reconstruction route: the registers already hold S_{t-1}, records folded)
    const float gc = FORM == kMamba2 ? G : alpha * gs;
    const float ge = FORM == kMamba2 ? 1.0f : alpha;
    const float* u = FORM == kMamba2 ? s.v : s.u;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const float ur = u[r * RPP + rg];
#pragma unroll
        for (int c = 0; c < VEC; ++c) cf[r][c] = gc * cf[r][c] + ur * kv[c];
    }
    // fp16 state and records: the records' rank-w update on the matrix
    // cores.  With D = the 16 x 16 block whose element (m, n) is tile row
    // 16 (R0 + m % 4) + 4 wave + m / 4 and column 8 n + c, each lane's block
    // elements are exactly its registers cf[R0 .. R0 + 3][c] (the layout of
    // v_mfma_f32_16x16x16_f16: lane l holds D rows 4 (l / 16) + i, column
    // l % 16), so the update accumulates in place.  The records' weighted
    // values f = e_j x_j (fp32) enter as fp16 pairs hi + lo with
    // hi = fp16(f), lo = fp16(f - hi) (two passes, |f - hi - lo| <= 2^-22 |f|
    // in fp16's normal range), the keys as they are stored (fp16); products
    // are exact and sums fp32.  |f| <= |x_j| (weights <= 1), so hi never
    // overflows.
    constexpr bool MF = std::is_same<TS, tF16>::value && std::is_same<TR, tF16>::value && !TWO && DK == 128 &&
                        LPR == 16 && RPP == 16 && NR % 4 == 0 && VEC == 8 && HPC == 1;
    if constexpr (MF) {
        typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
        typedef float f4_t __attribute__((ext_vector_type(4)));
        const int l = tid & 63;
        const int kq = 4 * (l >> 4);  // this lane's 4 of the block's 16 records (operands A and B)
        const int arow = 16 * (l & 3) + 4 * (tid >> 6) + ((l & 15) >> 2);  // its operand-A row, R0 = 0
        for (int jc = 0; jc < wd; jc += 16) {
            h4_t bk[VEC];  // keys: bk[c][i] = k_{jc + kq + i}[8 cc + c]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = jc + kq + i;
                u32x4 kw = u32x4{0u, 0u, 0u, 0u};
                if (j < wd) kw = *reinterpret_cast<const u32x4*>(s.k + (int64_t)j * DK + col0);
                _Float16 kh[VEC];
                __builtin_memcpy(kh, &kw, 16);
#pragma unroll
                for (int c = 0; c < VEC; ++c) bk[c][i] = kh[c];
            }
#pragma unroll
            for (int R0 = 0; R0 < NR; R0 += 4) {
                h4_t ahi, alo;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = jc + kq + i;
                    float f = 0.f;
                    if (j < wd) f = ge * s.e[j] * (float)s.x[(int64_t)j * DVW + 16 * R0 + arow];
                    const _Float16 hi = (_Float16)f;
                    ahi[i] = hi;
                    alo[i] = (_Float16)(f - (float)hi);
                }
#pragma unroll
                for (int c = 0; c < VEC; ++c) {
                    f4_t acc = {cf[R0][c], cf[R0 + 1][c], cf[R0 + 2][c], cf[R0 + 3][c]};
                    acc = __builtin_amdgcn_mfma_f32_16x16x16f16(ahi, bk[c], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x16f16(alo, bk[c], acc, 0, 0, 0);
                    cf[R0][c] = acc[0];
                    cf[R0 + 1][c] = acc[1];
                    cf[R0 + 2][c] = acc[2];
                    cf[R0 + 3][c] = acc[3];
                }
            }
        }
    } else {
        for (int j = 0; j < wd; ++j) {
            float kj[VEC];
            const R* kr = s.k + (int64_t)j * DK + col0;
#pragma unroll
            for (int h = 0; h < HPC; ++h) load_f<TR, EPC>(kr + EPC * LPR * h, kj + h * EPC);
            const float ej = ge * s.e[j];
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const float f = ej * to_f<TR>(s.x[(int64_t)j * DVW + r * RPP + rg]);
#pragma unroll
                for (int c = 0; c < VEC; ++c) cf[r][c] += f * kj[c];
            }
        }
    }
    if constexpr (std::is_same<TS, tF16>::value) {
        if (p.sr) {
            sr_store_rows<NR, HPC, LPR>(cf, ck + (int64_t)rg * DK + col0, p, id.tile, row0 + rg, RPP, DK, col0);
            if constexpr (TWO) {
#pragma unroll
                for (int r = 0; r < NR; ++r)
                    store_read_row<TL, VEC, LPR>(cf[r], cl + (int64_t)(r * RPP + rg) * DK + cc * VEC,
                                                 cs + r * RPP + rg, cc);
            }
            return;
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int64_t rowoff = (int64_t)(r * RPP + rg) * DK;
        u32x4 hp[HPC];
        pack_n<TS, VEC>(cf[r], hp);
        S* rowp = ck + rowoff + col0;
#pragma unroll
        for (int h = 0; h < HPC; ++h) st_stream(rowp + EPC * LPR * h, hp[h]);
        if constexpr (TWO) store_read_row<TL, VEC, LPR>(cf[r], cl + rowoff + cc * VEC, cs + r * RPP + rg, cc);
    }
}

// One tile, loads then arithmetic.
template <int FORM, int DV, int DK, class TS, class TR, class TI, int SPLIT, class TL, bool RECON, int ROWS,
          bool DEFER>
__device__ __forceinline__ void replay_tile(const StepParams& p, const TileIds id, char* smem, char* dslot) {
    // Without a flag array the (always present) cursor array is read in its
    // place and the result discarded, so that the load is unconditional.
    const uint8_t* fsrc = p.flush ? p.flush : reinterpret_cast<const uint8_t*>(p.write_pos);
    const bool flag = row_flag(fsrc, id.row) && p.flush;
    const int blk = p.block_table[id.row];
    const int word = p.write_pos[id.row];
    const int w = cursor_of(word);
    bool fl;
    TileIn<FORM, DV, DK, TS, TR, TI, SPLIT, TL, ROWS> in;
    in.run = tile_runs<ROWS>(p, id, blk, w, flag, fl);
    if (in.run) {
        tile_issue_small(p, id, blk, w, fl, zero_ckpt_of(word), in);
        tile_issue_stream(p, in);
    }
    tile_finish<FORM, DV, DK, TS, TR, TI, SPLIT, TL, RECON, ROWS, DEFER>(p, in, smem, dslot);
}

// Store the n deferred tiles at dbase, 16 bytes per thread and step.
template <int DV, int DK, class R, int SPLIT>
__device__ __forceinline__ void drain_deferred(const StepParams& p, char* dbase, int n) {
    constexpr int DVW = DV / SPLIT;
    using D = Deferred<DVW, DK, R>;
    constexpr int OCH = D::OUT / 16, KCH = D::KB / 16, XCH = D::XB / 16, CPE = OCH + KCH + XCH + 1;
    for (int c = threadIdx.x; c < n * CPE; c += blockDim.x) {
        const int e = c / CPE, j = c - e * CPE;
        char* ent = dbase + e * D::BYTES;
        const D df(ent);
        const int word = df.meta[2];
        if (word < 0) continue;
        const int w = cursor_of(word);
        const int tile = df.meta[0] / SPLIT, part = df.meta[0] - tile * SPLIT, blk = df.meta[1];
        const int row = tile / p.n_heads, head = tile - row * p.n_heads;
        char* base = p.pool + (int64_t)blk * p.block_bytes;
        if (j < OCH) {
            st_stream(reinterpret_cast<u32x4*>(p.out + (int64_t)tile * DV + part * DVW) + j,
                      reinterpret_cast<const u32x4*>(df.out)[j]);
        } else if (j < OCH + KCH) {
            const int grp = head / p.heads_per_group;
            if (part == 0 && head == grp * p.heads_per_group) {
                R* rk = reinterpret_cast<R*>(base + p.reck_off) + ((int64_t)grp * p.slots + w) * DK;
                st_stream(reinterpret_cast<u32x4*>(rk) + (j - OCH), reinterpret_cast<const u32x4*>(df.k)[j - OCH]);
            }
        } else if (j < OCH + KCH + XCH) {
            R* rx = reinterpret_cast<R*>(base + p.recx_off) + ((int64_t)head * p.slots + w) * DV + part * DVW;
            st_stream(reinterpret_cast<u32x4*>(rx) + (j - OCH - KCH), reinterpret_cast<const u32x4*>(df.x)[j - OCH - KCH]);
        } else if (part == 0) {
            st_nt(reinterpret_cast<float*>(base + p.reclam_off) + (int64_t)head * p.slots + w, *df.lam);
            if (head == 0 && p.next_wp)  // (non-flush rows only)
                st_nt(p.next_wp + row, (w + 1) | (word & RS_CURSOR_ZERO_CKPT));
        }
    }
}

// PERSIST (non-flush rows only): a one-dimensional grid of a few workgroups
// per compute unit, each taking the work items (tile * SPLIT + part)
// blockIdx.x, blockIdx.x + gridDim.x, ...  It first stages the items that
// run (in order, with their rows' block and cursor) in LDS at p.meta_off,
// then issues each item's loads ahead of the item before it, so that two
// workgroups per compute unit keep enough bytes in flight.  The outputs and
// appended records wait in LDS (p.defer_cap items from byte p.defer_off) and
// are stored after the workgroup's last item (or when full), so that the
// step's small writes follow the checkpoint stream instead of being
// interleaved with it.  Measured on MI355X: ~640 bytes of writes per 32 KiB
// tile read cost a 1 GiB read stream about 26 us when interleaved and about
// 6 us as one burst at the end; on the Nemotron-3-Super layer at batch 256
// this form takes the non-flush steps from 183-212 to 170-201 us (A/B
// harness, back-to-back launches).
template <int FORM, int DV, int DK, class TS, class TR, class TI, int SPLIT, class TL, bool RECON = false,
          int ROWS = kAllRows, bool PERSIST = false>
__global__ __launch_bounds__((StepTile<DV, DK, TL, SPLIT, ROWS>::NT),
                             1)
void k_replay_step(const StepParams p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    if constexpr (!PERSIST) {
        replay_tile<FORM, DV, DK, TS, TR, TI, SPLIT, TL, RECON, ROWS, false>(p, tile_ids<SPLIT>(p), smem, smem);
    } else {
        using R = typename TR::S;
        using D = Deferred<DV / SPLIT, DK, R>;
        using In = TileIn<FORM, DV, DK, TS, TR, TI, SPLIT, TL, ROWS>;
        constexpr int NT = StepTile<DV, DK, TL, SPLIT, ROWS>::NT;
        const int G = (int)gridDim.x;
        const int items = p.n_rows * p.n_heads * SPLIT;
        const int mine = (items - (int)blockIdx.x + G - 1) / G;  // >= 1: the grid is at most the items
        auto ids = [&](int t) {
            TileIds id;
            id.tile = t / SPLIT;
            id.part = t - (int)id.tile * SPLIT;
            id.row = (int)id.tile / p.n_heads;
            id.head = (int)id.tile - id.row * p.n_heads;
            return id;
        };
        // Staging: the items of this workgroup that run, in order, each with
        // its row's block and cursor (3 ints), after an error counter, the
        // running count and one total per wave.
        int* err_lds = reinterpret_cast<int*>(smem + p.meta_off);
        int* cnt_lds = err_lds + 1;
        int* wave_n = err_lds + 4;
        int* list = err_lds + 8;
        static_assert(NT / 64 <= 4, "wave totals");
        if (threadIdx.x == 0) *err_lds = *cnt_lds = 0;
        __syncthreads();
        for (int c = 0; c < mine; c += NT) {
            const int i = c + (int)threadIdx.x;
            const int t = (int)blockIdx.x + i * G;
            int blk = -1, w = 0;
            bool run = false;
            if (i < mine) {
                const TileIds id = ids(t);
                blk = p.block_table[id.row];
                w = p.write_pos[id.row];  // the cursor word (RS_CURSOR_ZERO_CKPT kept)
                const bool flag = p.flush && row_flag(p.flush, id.row);
                bool fl;
                run = tile_runs<ROWS, true>(p, id, blk, cursor_of(w), flag, fl, err_lds);
            }
            const uint64_t ball = __ballot(run);
            const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
            if (lane == 0) wave_n[wave] = __popcll(ball);
            __syncthreads();
            int k = *cnt_lds + __popcll(ball & ((1ull << lane) - 1));
            for (int v = 0; v < wave; ++v) k += wave_n[v];
            if (run) {
                list[3 * k] = t;
                list[3 * k + 1] = blk;
                list[3 * k + 2] = w;
            }
            __syncthreads();
            if (threadIdx.x == 0)
                for (int v = 0; v < NT / 64; ++v) *cnt_lds += wave_n[v];
            __syncthreads();
        }
        const int cnt = __builtin_amdgcn_readfirstlane(*cnt_lds);
        // running item j (in scalar registers: the branches on them are uniform)
        auto issue = [&](int j, In& in) {
            const int t = __builtin_amdgcn_readfirstlane(list[3 * j]);
            const int blk = __builtin_amdgcn_readfirstlane(list[3 * j + 1]);
            const int w = __builtin_amdgcn_readfirstlane(list[3 * j + 2]);
            tile_issue_small<FORM, DV, DK, TS, TR, TI, SPLIT, TL, ROWS, true>(p, ids(t), blk, cursor_of(w), false,
                                                                           zero_ckpt_of(w), in);
        };
        char* dbase = smem + p.defer_off;
        int n = 0;
        // Consecutive items use the two halves of the records area in turn
        // (a: the first, b: the second), so an item's LDS is free again once
        // the next item has passed its own barriers and no barrier is needed
        // between items; one comes before every drain.
        const int carve = (int)((lds_need<DV / SPLIT, DK, R>(p.slots, p.L) + 15) / 16 * 16);
        auto finish = [&](const In& in, int half) {
            tile_finish<FORM, DV, DK, TS, TR, TI, SPLIT, TL, RECON, ROWS, true>(p, in, smem + half * carve,
                                                                                 dbase + n * D::BYTES);
            if (++n == p.defer_cap) {
                __syncthreads();  // the items' deferred writes are visible
                drain_deferred<DV, DK, R, SPLIT>(p, dbase, n);
                n = 0;
                // Wait for the drain's stores here: a global write still
                // pending at the loop's next waits would make the compiler
                // wait for every outstanding load there, the prefetched ones
                // included (vmcnt(0) only; the other counters are left).
                __builtin_amdgcn_s_waitcnt(0x0F70);
                __syncthreads();
            }
        };
        // Two sets of loads that trade places (no register copies, which
        // would wait for the loads): item j's small loads are issued two
        // items ahead and its stream one item ahead, so that the loads an
        // item waits for are all older than the next item's.  The steady
        // loop has no branch around a load and issues in the same order as
        // the prologue (small a, stream a, small b), so that the compiler's
        // waits there count exactly; the last one to three items follow it.
        if (cnt > 0) {
            In a, b;
            issue(0, a);
            tile_issue_stream(p, a, true);
            issue(min(1, cnt - 1), b);
            int j = 0;
            for (; j + 3 < cnt; j += 2) {
                tile_issue_stream(p, b, true);
                finish(a, 0);
                issue(j + 2, a);
                tile_issue_stream(p, a, true);
                finish(b, 1);
                issue(j + 3, b);
            }
            // items j .. cnt - 1: a (small and stream issued), b (small issued)
            if (j + 1 < cnt) tile_issue_stream(p, b, true);
            finish(a, 0);
            if (j + 2 < cnt) {
                issue(j + 2, a);
                tile_issue_stream(p, a, true);
            }
            if (j + 1 < cnt) finish(b, 1);
            if (j + 2 < cnt) finish(a, 0);
        }
        __syncthreads();  // the items' deferred writes are visible
        drain_deferred<DV, DK, R, SPLIT>(p, dbase, n);
        if (threadIdx.x == 0 && *err_lds && p.err) atomicAdd(p.err, *err_lds);
    }
}

// ------------------------------------------------ conventional decode step --
template <int FORM, int DV, int DK, class TS, class TI, int SPLIT>
__global__ __launch_bounds__((Tile<DV, DK, TS, SPLIT>::NT)) void k_conventional_step(const StepParams p) {
    using T = Tile<DV, DK, TS, SPLIT>;
    using S = typename TS::S;
    using I = typename TI::S;
    constexpr int VEC = T::VEC, LPR = T::LPR, RPP = T::RPP, NR = T::NR, DVW = T::DVW;
    constexpr int KEEP = FORM == kGdn ? 2 : 1;
    constexpr int NV = KEEP * NR;

    const TileIds id = tile_ids<SPLIT>(p);
    const int blk = p.block_table[id.row];
    if (blk < 0) return;
    if (blk >= p.n_blocks) {
        count_error(p, id);
        return;
    }
    const int tid = threadIdx.x;
    const int cc = tid % LPR;
    const int rg = tid / LPR;
    const int row0 = id.part * DVW;

    char* base = p.pool + (int64_t)blk * p.block_bytes;
    S* ck = reinterpret_cast<S*>(base + p.ckpt_off) + (int64_t)id.head * (DV * DK) + (int64_t)row0 * DK;
    const int grp = id.head / p.heads_per_group;
    const I* qp = static_cast<const I*>(p.q) + id.row * p.qs_r + grp * p.qs_h;
    const I* kp = static_cast<const I*>(p.k) + id.row * p.ks_r + grp * p.ks_h;
    const I* vp = static_cast<const I*>(p.v) + id.row * p.vs_r + id.head * p.vs_h + row0;

    __shared__ float s_v[DVW], s_u[DVW];

    float qv[VEC], kv[VEC];
    load_f<TI, VEC>(qp + cc * VEC, qv);
    load_f<TI, VEC>(kp + cc * VEC, kv);
    const float vi = to_f<TI>(vp[min(tid, DVW - 1)]);
    u32x4 cb[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) cb[r] = ld_stream(ck + (int64_t)(r * RPP + rg) * DK + cc * VEC);
    const float alpha = expf(p.lam[id.tile]);
    const float bt = FORM == kGdn ? p.beta[id.tile] : 0.f;  // loaded with the others, used at the end
    if (tid < DVW) s_v[tid] = vi;

    float kq = 0.f;
#pragma unroll
    for (int c = 0; c < VEC; ++c) kq += kv[c] * qv[c];
    kq = group_sum<LPR>(kq);
    __syncthreads();

    // o = S_t q = alpha (S_{t-1} q) + (k . q) u, with u = v (Mamba-2) or the
    // corrected value d = beta (v - alpha S_{t-1} k) (Gated DeltaNet).
    float cf[NR][VEC];
#pragma unroll
    for (int r = 0; r < NR; ++r) unpack16<TS>(cb[r], cf[r]);
    float acc[NV];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            a += cf[r][c] * qv[c];
            if constexpr (FORM == kGdn) b += cf[r][c] * kv[c];
        }
        if constexpr (FORM == kMamba2) {
            acc[r] = alpha * a;
            if (cc == LPR - 1) acc[r] += kq * s_v[r * RPP + rg];
        } else {
            acc[2 * r] = a;
            acc[2 * r + 1] = b;
        }
    }
    xsum<NV, LPR / 2, KEEP>(acc, cc);
    float* o = p.out + id.tile * DV + row0;
    {
        constexpr int left = xsum_left<NV, LPR, KEEP>();
        const int b0 = xsum_base<NV, LPR, KEEP>(cc);
        if ((cc & xsum_dup_mask<NV, LPR, KEEP>()) == 0) {
            if constexpr (FORM == kMamba2) {
#pragma unroll
                for (int i = 0; i < left; ++i) st_nt(o + (b0 + i) * RPP + rg, acc[i]);
            } else {
#pragma unroll
                for (int i = 0; i < left; i += 2) {
                    const int row = ((b0 + i) / 2) * RPP + rg;
                    const float d = bt * (s_v[row] - alpha * acc[i + 1]);
                    st_nt<kNtSmall<FORM>>(o + row, alpha * acc[i] + kq * d);
                    s_u[row] = d;
                }
            }
        }
    }
    if constexpr (FORM == kGdn) __syncthreads();  // d in LDS

    // S_t = alpha S_{t-1} + u k^T, stored every step.
    const float* u = FORM == kMamba2 ? s_v : s_u;
    if constexpr (std::is_same<TS, tF16>::value) {
        if (p.sr) {
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const float ur = u[r * RPP + rg];
#pragma unroll
                for (int c = 0; c < VEC; ++c) cf[r][c] = alpha * cf[r][c] + ur * kv[c];
            }
            sr_store_rows<NR, 1, LPR>(cf, ck + (int64_t)rg * DK + cc * VEC, p, id.tile, row0 + rg, RPP, DK, cc * VEC);
            return;
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const float ur = u[r * RPP + rg];
#pragma unroll
        for (int c = 0; c < VEC; ++c) cf[r][c] = alpha * cf[r][c] + ur * kv[c];
        st_stream(ck + (int64_t)(r * RPP + rg) * DK + cc * VEC, pack16<TS>(cf[r]));
    }
}

// ------------------------------------------------------ token-less flush --
// Fold the w buffered records into the (recurrence) checkpoint; with a
// two-precision checkpoint the read copy is rewritten from the same values.
template <int DV, int DK, class TS, class TR, int SPLIT, class TL>
__global__ __launch_bounds__((Tile<DV, DK, TL, SPLIT>::NT)) void k_replay_flush(const StepParams p) {
    using T = Tile<DV, DK, TL, SPLIT>;
    using S = typename TS::S;
    using RL = typename TL::S;
    using R = typename TR::S;
    constexpr int NT = T::NT, VEC = T::VEC, LPR = T::LPR, RPP = T::RPP, NR = T::NR, DVW = T::DVW;
    constexpr bool TWO = !std::is_same<TS, TL>::value;
    constexpr int HPC = VEC * (int)sizeof(S) / 16;  // lane order as in k_replay_step
    constexpr int EPC = VEC / HPC;

    const TileIds id = tile_ids<SPLIT>(p);
    const bool flag = row_flag(p.flush, id.row);
    const int blk = p.block_table[id.row];
    const int word = p.write_pos[id.row];
    const int w = cursor_of(word);
    const bool zc = zero_ckpt_of(word);  // the checkpoint is zero: not read, written as the fold
    if (blk < 0 || !flag) return;
    if (blk >= p.n_blocks || w < 0 || w > p.slots) {
        count_error(p, id);
        return;
    }
    if (w == 0 && !zc) return;  // nothing buffered: the checkpoint is the state

    const int tid = threadIdx.x;
    const int cc = tid % LPR;
    const int rg = tid / LPR;
    const int row0 = id.part * DVW;
    char* base = p.pool + (int64_t)blk * p.block_bytes;
    S* ck = reinterpret_cast<S*>(base + p.ckpt_off) + (int64_t)id.head * (DV * DK) + (int64_t)row0 * DK;
    RL* cl = reinterpret_cast<RL*>(base + p.ckpt_lo_off) + (int64_t)id.head * (DV * DK) + (int64_t)row0 * DK;
    float* cs = reinterpret_cast<float*>(base + p.ckpt_sc_off) + id.head * DV + row0;
    const R* rx = reinterpret_cast<const R*>(base + p.recx_off) + (int64_t)id.head * p.slots * DV + row0;
    const R* rk =
        reinterpret_cast<const R*>(base + p.reck_off) + (int64_t)(id.head / p.heads_per_group) * p.key_slots * DK;
    const float* rl = reinterpret_cast<const float*>(base + p.reclam_off) + (int64_t)id.head * p.slots;

    extern __shared__ __attribute__((aligned(16))) char smem[];
    const Lds<R> s = carve<DVW, DK, R>(smem, p.slots, p.L);

    const int col0 = EPC * cc;
    auto col = [col0](int h) { return col0 + EPC * LPR * h; };
    const float lam_j = w > 0 ? rl[min(tid, w - 1)] : 0.f;
    RecordCopy<DV, DVW, DK, R, NT, 2> rec;
    rec.issue(rk, rx, w);
    u32x4 cb[NR * HPC];
    if (!zc) {
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int h = 0; h < HPC; ++h) cb[r * HPC + h] = ld_stream(ck + (int64_t)(r * RPP + rg) * DK + col(h));
    } else {
#pragma unroll
        for (int i = 0; i < NR * HPC; ++i) cb[i] = u32x4{0u, 0u, 0u, 0u};
    }
    rec.commit(rk, rx, s.k, s.x);
    decay_weights(lam_j, s.e, s.sc, w, 0.0f);
    __syncthreads();

    // C' = G C + sum_j e_j x_j k_j^T  with G = exp(sum_{l<w} lam_l).
    const float G = s.sc[0];
    float cf[NR][VEC];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        unpack_n<TS, VEC>(&cb[r * HPC], cf[r]);
#pragma unroll
        for (int c = 0; c < VEC; ++c) cf[r][c] *= G;
    }
    for (int j = 0; j < w; ++j) {
        float kj[VEC];
#pragma unroll
        for (int h = 0; h < HPC; ++h) load_f<TR, EPC>(s.k + (int64_t)j * DK + col(h), kj + h * EPC);
        const float ej = s.e[j];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const float f = ej * to_f<TR>(s.x[(int64_t)j * DVW + r * RPP + rg]);
#pragma unroll
            for (int c = 0; c < VEC; ++c) cf[r][c] += f * kj[c];
        }
    }
    if constexpr (std::is_same<TS, tF16>::value) {
        if (p.sr) {
            sr_store_rows<NR, HPC, LPR>(cf, ck + (int64_t)rg * DK + col0, p, id.tile, row0 + rg, RPP, DK, col0);
            if constexpr (TWO) {
#pragma unroll
                for (int r = 0; r < NR; ++r)
                    store_read_row<TL, VEC, LPR>(cf[r], cl + (int64_t)(r * RPP + rg) * DK + cc * VEC,
                                                 cs + r * RPP + rg, cc);
            }
            return;
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int64_t rowoff = (int64_t)(r * RPP + rg) * DK;
        u32x4 hp[HPC];
        pack_n<TS, VEC>(cf[r], hp);
#pragma unroll
        for (int h = 0; h < HPC; ++h) st_stream(ck + rowoff + col(h), hp[h]);
        if constexpr (TWO) store_read_row<TL, VEC, LPR>(cf[r], cl + rowoff + cc * VEC, cs + r * RPP + rg, cc);
    }
}

// ------------------------------------------------ speculative verify step --
// One workgroup per (row, head) tile (split 1 only: a flushing row rewrites
// record slots 0..T-1 that it has just read, which another workgroup of the
// same tile could still be reading).  T draft tokens per row.  Order of work:
//   1. small loads (draft q, k, v and log-decays, the committed records and
//      their decays), then the checkpoint stream;
//   2. drafts and records to LDS; barrier; log-decay sums of the committed
//      records (suffix sums, wave 0) and of the drafts (prefix sums); barrier;
//   3. K^T Q: lane group rg takes keys rg, rg + RPP, ... (committed records,
//      then drafts) against all T queries, one lane-group reduction per key;
//      each (key, query) product is scaled by its decay weight, zero where a
//      draft comes after the query (the causal mask); barrier;
//   4. per lane: T x NR partial sums of the checkpoint GEMV for all T queries
//      plus this lane's share of the weighted record and draft terms, then
//      one lane-group reduction yielding the T output rows;
//   5. flush rows fold the committed records into the registers holding the
//      tile and store it once; every row stores its drafts as records behind
//      the committed ones (from slot 0 after a flush).
// Every decay weight is the exponential of a sum of log-decays (<= 0).
template <class R>
struct SpecLds {
    R* kc;        // [slots][DK] committed keys
    R* xc;        // [slots][DV] committed values
    float* qd;    // [T][DK] draft queries
    float* kd;    // [T][DK] draft keys
    float* vd;    // [T][DV] draft values
    float* lamd;  // [T] draft log-decays
    float* lsc;   // [slots] sum of the committed log-decays after record j
    float* ec;    // [slots] exp(lsc)
    float* cum;   // [T] sum of the draft log-decays 1..i
    float* gck;   // [T] checkpoint weight of draft i
    float* wq;    // [(slots + T) * T] weighted key . query products
    float* sc;    // [4] total committed log-decay, its exponential
};

template <int DV, int DK, class R>
__device__ __forceinline__ SpecLds<R> spec_carve(char* smem, int slots, int T) {
    SpecLds<R> s;
    s.kc = reinterpret_cast<R*>(smem);
    s.xc = s.kc + (int64_t)slots * DK;
    float* f = reinterpret_cast<float*>(s.xc + (int64_t)slots * DV);
    s.qd = f;
    s.kd = s.qd + T * DK;
    s.vd = s.kd + T * DK;
    s.lamd = s.vd + T * DV;
    s.lsc = s.lamd + T;
    s.ec = s.lsc + slots;
    s.cum = s.ec + slots;
    s.gck = s.cum + T;
    s.wq = s.gck + T;
    s.sc = s.wq + (slots + T) * T;
    return s;
}

size_t spec_lds_bytes(int slots, int T, int dv, int dk, int rec_bytes) {
    return (size_t)slots * (dk + dv) * rec_bytes +
           sizeof(float) * (2 * (size_t)T * dk + (size_t)T * dv + T + 2 * (size_t)slots + 2 * (size_t)T +
                            ((size_t)slots + T) * T + 4);
}

// Raw 4-element load (io type) into 32-bit words; the conversion to float
// happens when the words are used, so the load does not wait.
template <class TI>
struct Raw4 {
    static constexpr int W = 4 * (int)sizeof(typename TI::S) / 4;
    uint32_t w[W];
    __device__ __forceinline__ void load(const typename TI::S* p) {
        if constexpr (W == 4) {
            const u32x4 r = *reinterpret_cast<const u32x4*>(p);
            w[0] = r[0]; w[1] = r[1]; w[2] = r[2]; w[3] = r[3];
        } else {
            const u32x2 r = *reinterpret_cast<const u32x2*>(p);
            w[0] = r[0]; w[1] = r[1];
        }
    }
    __device__ __forceinline__ void to(float* out) const {
        typename TI::S tmp[4];
        __builtin_memcpy(tmp, w, sizeof(tmp));
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = to_f<TI>(tmp[i]);
    }
};

// Four consecutive elements of a read copy: 8 bytes of fp16 / bf16, or 4
// bytes of E4M3 codes whose row scale the caller applies (speculative verify
// over a two-precision checkpoint, one lane's four columns of a row).
template <class TL>
struct Quad {
    using RL = typename TL::S;
    using W = typename std::conditional<sizeof(RL) == 2, u32x2, uint32_t>::type;
    W w;
    __device__ __forceinline__ void load(const RL* p) { w = __builtin_nontemporal_load(reinterpret_cast<const W*>(p)); }
    __device__ __forceinline__ void to(float* out, float scale) const {
        if constexpr (kScaled<TL>) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
            out[0] = lo[0] * scale;
            out[1] = lo[1] * scale;
            out[2] = hi[0] * scale;
            out[3] = hi[1] * scale;
        } else {
            RL tmp[4];
            __builtin_memcpy(tmp, &w, sizeof(tmp));
#pragma unroll
            for (int i = 0; i < 4; ++i) out[i] = to_f<TL>(tmp[i]);
        }
    }
};

// Store four values of a read-copy row, rounded to nearest even; E4M3: the
// row (G lanes, 4 values each) shares one power-of-two scale, chosen as in
// encode_e4m3_row, which lane 0 of the group stores.
template <class TL, int G>
__device__ __forceinline__ void store_read_quad(const float* x, typename TL::S* dst, float* scale, int lane_in_row) {
    using W = typename Quad<TL>::W;
    W w;
    if constexpr (kScaled<TL>) {
        float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
        group_max<G>(amax);
        const uint32_t b = __float_as_uint(amax);
        int e = (int)((b >> 23) & 0xffu) - 127 - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
        e = max(e, -100);
        int c = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(x[0], -e), __builtin_amdgcn_ldexpf(x[1], -e), 0,
                                                false);
        c = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(x[2], -e), __builtin_amdgcn_ldexpf(x[3], -e), c, true);
        w = (uint32_t)c;
        if (lane_in_row == 0) st_nt(scale, __builtin_amdgcn_ldexpf(1.0f, e));
    } else {
        typename TL::S tmp[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) tmp[i] = from_f<TL>(x[i]);
        __builtin_memcpy(&w, tmp, sizeof(tmp));
    }
    __builtin_nontemporal_store(w, reinterpret_cast<W*>(dst));
}

// Whether the speculative verify runs its state products on the matrix
// cores: an fp32 state whose d_v rows fill four waves' 16-row blocks and
// whose d_k columns come in 16-column slices, at the draft counts where that
// measured faster (batch 256: Gated DeltaNet T = 4 and 8, Mamba-2 T = 8; at
// fewer drafts the T (Mamba-2) or 2T columns fill a fraction of each 16-column
// product: Mamba-2 at T = 4 and Gated DeltaNet at T = 2 were 7-12 % and 5-10 %
// slower than the VALU form).
constexpr bool spec_mf(int form, int dv, int dk, bool f32_state, int T) {
    return f32_state && dv % 64 == 0 && dk % 16 == 0 && (size_t)dv * dk / 4 / 4 >= 256 &&
           (form == kGdn ? T >= 4 : T == 8);
}

// TL != TS: a two-precision checkpoint (fp32 recurrence copy TS, read copy
// TL; blog "The precision argument, derived").  A row that does not flush
// reads only the read copy for its outputs; a flushing row reads the
// recurrence copy, folds in fp32 and stores both copies from the same
// unrounded values.  The read copy keeps the lane order of the standard
// step's layout (rs_block_layout): this lane's four columns 4 cc .. 4 cc + 3
// sit at position n (cc mod (DK / n)) + 4 (cc div (DK / n)) of the row, n
// read elements per 16 bytes.
template <int DV, int DK, class TS, class TR, class TI, int T, class TL = TS>
__global__ __launch_bounds__((Tile<DV, DK, TS, 1>::NT)) void k_spec_verify(const StepParams p) {
    using Tl = Tile<DV, DK, TS, 1>;
    using S = typename TS::S;
    using R = typename TR::S;
    using I = typename TI::S;
    using RL = typename TL::S;
    constexpr bool TWO = !std::is_same<TS, TL>::value;
    constexpr bool SC = kScaled<TL>;
    static_assert(!TWO || std::is_same<TS, tF32>::value, "a read copy under an fp32 recurrence copy");
    constexpr int NT = Tl::NT, VEC = Tl::VEC, LPR = Tl::LPR, RPP = Tl::RPP, NR = Tl::NR;
    constexpr int NV = T * NR;                        // partial sums per lane: (draft, owned row)
    constexpr bool MF = !TWO && spec_mf(kMamba2, DV, DK, std::is_same<TS, tF32>::value, T);
    constexpr int QN = (T * DK / 4 + NT - 1) / NT;    // 4-element pieces of draft q / k per thread
    constexpr int VN = (T * DV + NT - 1) / NT;        // draft v elements per thread
    constexpr int KCH = DK * (int)sizeof(R) / 16, XCH = DV * (int)sizeof(R) / 16, XE = 16 / (int)sizeof(R);
    constexpr int RC = 2;                             // record chunks per thread in registers
    static_assert(DK % 4 == 0 && VEC % 4 == 0, "4-element pieces");

    const TileIds id = tile_ids<1>(p);
    const uint8_t* fsrc = p.flush ? p.flush : reinterpret_cast<const uint8_t*>(p.write_pos);
    const bool flag = row_flag(fsrc, id.row) && p.flush;
    const int blk = p.block_table[id.row];
    const int h = p.write_pos[id.row];
    const bool pad = blk < 0;
    const bool bad = !pad && (blk >= p.n_blocks || h < 0 || h > p.slots);
    if (pad || bad) {
        if (bad) count_error(p, id);
        return;
    }
    const bool fl = flag || (h + T > p.L);  // no room for T more records: flush first
    const int base = fl ? 0 : h;            // slot of this step's first draft
    const int tid = threadIdx.x;
    const int cc = tid % LPR;
    const int rg = tid / LPR;
    // keys and queries per group of heads_per_group heads (1: per head); the
    // group's first head stores its draft keys, a flushing row's in the
    // staging slots (the other heads may still read the committed ones)
    const int grp = id.head / p.heads_per_group;
    const bool key_owner = id.head == grp * p.heads_per_group;
    const int kbase = fl && p.heads_per_group > 1 ? p.slots : base;

    char* bp = p.pool + (int64_t)blk * p.block_bytes;
    S* ck = reinterpret_cast<S*>(bp + p.ckpt_off) + (int64_t)id.head * (DV * DK);
    R* rx = reinterpret_cast<R*>(bp + p.recx_off) + (int64_t)id.head * p.slots * DV;
    R* rk = reinterpret_cast<R*>(bp + p.reck_off) + (int64_t)grp * p.key_slots * DK;
    float* rl = reinterpret_cast<float*>(bp + p.reclam_off) + (int64_t)id.head * p.slots;
    const I* qb = static_cast<const I*>(p.q) + id.row * p.qs_r + grp * p.qs_h;
    const I* kb = static_cast<const I*>(p.k) + id.row * p.ks_r + grp * p.ks_h;
    const I* vb = static_cast<const I*>(p.v) + id.row * p.vs_r + id.head * p.vs_h;
    const int64_t tok0 = (int64_t)id.row * T;  // this row's first token in [row][T] arrays
    // read copy (two-precision checkpoint): this lane's columns in a row
    RL* cl = reinterpret_cast<RL*>(bp + p.ckpt_lo_off) + (int64_t)id.head * (DV * DK);
    float* cs = reinterpret_cast<float*>(bp + p.ckpt_sc_off) + (int64_t)id.head * DV;
    constexpr int RN = 16 / (int)sizeof(RL), RCH = DK / RN;  // read elements per 16 bytes, chunks per row
    const int lpos = RN * (cc % RCH) + 4 * (cc / RCH);
    static_assert(!TWO || (VEC == 4 && DK % RN == 0), "four fp32 columns per lane");

    extern __shared__ __attribute__((aligned(16))) char smem[];
    const SpecLds<R> s = spec_carve<DV, DK, R>(smem, p.slots, T);

    // 1. small loads, then the checkpoint stream
    Raw4<TI> qr[QN], kr[QN];
#pragma unroll
    for (int u = 0; u < QN; ++u) {
        const int e = min((u * NT + tid) * 4, T * DK - 4);  // clamped: every thread loads
        const int i = e / DK, c = e - i * DK;
        qr[u].load(qb + i * p.qs_t + c);
        kr[u].load(kb + i * p.ks_t + c);
    }
    I vr[VN];
#pragma unroll
    for (int u = 0; u < VN; ++u) {
        const int e = min(u * NT + tid, T * DV - 1);
        const int i = e / DV;
        vr[u] = vb[i * p.vs_t + (e - i * DV)];
    }
    const float lam_d = p.lam[(tok0 + min(tid, T - 1)) * p.n_heads + id.head];
    float lam_c = 0.f;
    if (h > 0) lam_c = rl[min(tid, h - 1)];
    // committed records: keys [h][DK] then values [h][DV], 16-byte chunks
    const int nk = h * KCH, nrec = nk + h * XCH;
    auto rsrc = [&](int i) -> const R* {
        if (i < nk) return rk + (int64_t)i * XE;
        const int t2 = i - nk, j = t2 / XCH;
        return rx + (int64_t)j * DV + (t2 - j * XCH) * XE;
    };
    auto rdst = [&](int i) -> u32x4* {
        return i < nk ? reinterpret_cast<u32x4*>(s.kc) + i : reinterpret_cast<u32x4*>(s.xc) + (i - nk);
    };
    u32x4 rb[RC];
    if (nrec > 0) {
#pragma unroll
        for (int u = 0; u < RC; ++u) rb[u] = ld_stream(rsrc(min(u * NT + tid, nrec - 1)));
    }
    // records beyond RC chunks per thread (long rings only) are copied before
    // the checkpoint stream is issued, so that waiting for them never waits
    // for the stream
    for (int i = RC * NT + tid; i < nrec; i += NT) *rdst(i) = ld_stream(rsrc(i));
    u32x4 cb[NR];
    Quad<TL> lq[NR];  // two-precision, a row that does not flush: the read copy instead
    float lsc[NR];
    // Matrix-core form: the load layout of k_spec_verify_gdn's (wave wv, its
    // 16-row blocks b, lane (rm, cg): row 16 (wv NB + b) + rm, columns
    // 16 q + 4 cg .. + 3), the A operand of the 16 x 16 x 4 fp32 product
    constexpr int NB = DV / 64, NP = DK / 16;
    [[maybe_unused]] const int wv = tid >> 6, rm = tid & 15, cg = (tid >> 4) & 3;
    if constexpr (MF) {
        static_assert(NB * NP == NR && NT == 256, "four waves of 16-row blocks");
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int q = 0; q < NP; ++q)
                cb[b * NP + q] = *reinterpret_cast<const u32x4*>(ck + (int64_t)(16 * (wv * NB + b) + rm) * DK + 16 * q + 4 * cg);
    } else if (!TWO || fl) {  // uniform
#pragma unroll
        for (int r = 0; r < NR; ++r) cb[r] = ld_stream(ck + (int64_t)(r * RPP + rg) * DK + cc * VEC);
    } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            lq[r].load(cl + (int64_t)(r * RPP + rg) * DK + lpos);
            lsc[r] = SC ? cs[r * RPP + rg] : 1.0f;
        }
    }

    // 2. to LDS
#pragma unroll
    for (int u = 0; u < QN; ++u) {
        const int e = (u * NT + tid) * 4;
        if (e < T * DK) {
            qr[u].to(s.qd + e);
            kr[u].to(s.kd + e);
        }
    }
#pragma unroll
    for (int u = 0; u < VN; ++u)
        if (u * NT + tid < T * DV) s.vd[u * NT + tid] = to_f<TI>(vr[u]);
    if (tid < T) s.lamd[tid] = lam_d;
#pragma unroll
    for (int u = 0; u < RC; ++u)
        if (u * NT + tid < nrec) *rdst(u * NT + tid) = rb[u];
    __syncthreads();

    if (tid < 64) {
        // committed records: lane j < h gets sum_{j<l<h} lam_l; lane 0 the total
        const int lane = tid;
        float sfx = lane < h ? lam_c : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {  // inclusive suffix sum over lanes >= lane
            const float t = __shfl_down(sfx, off);
            if (lane + off < 64) sfx += t;
        }
        float after = __shfl_down(sfx, 1);
        if (lane == 63) after = 0.f;
        if (lane < h) {
            s.lsc[lane] = after;
            s.ec[lane] = expf(after);
        }
        if (lane == 0) {
            s.sc[0] = sfx;
            s.sc[1] = expf(sfx);
        }
        if (lane < T) {  // drafts: sum of the log-decays 1..lane
            float c = 0.f;
            for (int m = 0; m <= lane; ++m) c += s.lamd[m];
            s.cum[lane] = c;
        }
    }
    __syncthreads();

    // 3. weighted K^T Q
    // The lane holds query i at position i ^ mq (mq from its lane-group
    // bits), so that the reductions over the query index need no selects
    // (xsum_perm); weights indexed by query are read at i ^ mq.
    constexpr int PL = xsum_perm_levels<T, LPR>();
    const int mq = xsum_perm_mask<T, LPR>(cc);
    float qv[T][VEC];
#pragma unroll
    for (int i = 0; i < T; ++i)
#pragma unroll
        for (int c = 0; c < VEC; ++c) qv[i][c] = s.qd[(i ^ mq) * DK + cc * VEC + c];
    if (tid < T) s.gck[tid] = expf(s.sc[0] + s.cum[tid]);
    const int nkeys = h + T;
    for (int j0 = 0; j0 < nkeys; j0 += RPP) {
        const int j = j0 + rg;
        float kj[VEC];
        if (j < h) {
            load_f<TR, VEC>(s.kc + (int64_t)j * DK + cc * VEC, kj);
        } else {
            const int m = min(j - h, T - 1);
#pragma unroll
            for (int c = 0; c < VEC; ++c) kj[c] = s.kd[m * DK + cc * VEC + c];
        }
        float part[T];
#pragma unroll
        for (int i = 0; i < T; ++i) {
            float a = 0.f;
#pragma unroll
            for (int c = 0; c < VEC; ++c) a += kj[c] * qv[i][c];
            part[i] = a;
        }
        xsum_perm<T, LPR / 2, PL>(part, cc);
        constexpr int left = xsum_left<T, LPR, 1>();
        if (j < nkeys && (cc & xsum_dup_mask<T, LPR, 1>()) == 0) {
            const int b0 = xsum_perm_base<T, LPR, T>(cc);
#pragma unroll
            for (int k = 0; k < left; ++k) {
                const int i = b0 + k;
                float wgt;
                if (j < h) {
                    wgt = expf(s.lsc[j] + s.cum[i]);
                } else {
                    const int m = j - h;
                    float sm = 0.f;
                    for (int l = m + 1; l <= i; ++l) sm += s.lamd[l];
                    wgt = m <= i ? expf(sm) : 0.f;  // drafts after query i are masked
                }
                s.wq[j * T + i] = wgt * part[k];
            }
        }
    }
    __syncthreads();

    if constexpr (MF) {
        using f4 = __attribute__((ext_vector_type(4))) float;
        f4 cf[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) cf[r] = __builtin_bit_cast(f4, cb[r]);
        // 4. O = C Qg + X Wq on the matrix cores: Qg = [g_1 q_1 .. g_T q_T]
        //    (d_k x T, zero beyond), X the committed values then the drafts'
        //    (x_j at row, column j), Wq the weighted key products; lane (rm,
        //    cg) ends with rows 4 cg .. + 3 of each block for draft n = rm
        const float* wsrc = s.qd + min(rm, T - 1) * DK + 4 * cg;
        const float wsc = rm < T ? s.gck[min(rm, T - 1)] : 0.f;
        f4 y[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) y[b] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const f4 w = *reinterpret_cast<const f4*>(wsrc + 16 * q) * wsc;
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int b = 0; b < NB; ++b) y[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(cf[b * NP + q][e], w[e], y[b], 0, 0, 0);
        }
        // committed records then drafts, four at a time; a slot past them
        // takes slot 0's (finite) value with weight zero
        for (int j0 = 0; j0 < nkeys; j0 += 4) {
            const int jj = j0 + cg;
            const int jc = jj < nkeys ? jj : 0;
            const float g = jj < nkeys && rm < T ? s.wq[jc * T + min(rm, T - 1)] : 0.f;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int row = 16 * (wv * NB + b) + rm;
                const float xa = jc < h ? to_f<TR>(s.xc[(int64_t)(jc < h ? jc : 0) * DV + row]) : s.vd[max(jc - h, 0) * DV + row];
                y[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa, g, y[b], 0, 0, 0);
            }
        }
        if (rm < T) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
                __builtin_nontemporal_store(
                    y[b], reinterpret_cast<f4*>(p.out + ((tok0 + rm) * p.n_heads + id.head) * DV + 16 * (wv * NB + b) + 4 * cg));
        }
        // 5. flush: C = G C + sum_j e_j x_j k_j^T on the matrix cores, in
        //    place (as C^T += K^T F^T: keys as A, F = e_j x_j as B; the
        //    product's rows 4 cg .. + 3 at column rm are the lane's four
        //    values of slice q), stored from where it was loaded
        if (fl) {  // uniform
            const float G = s.sc[1];
#pragma unroll
            for (int r = 0; r < NR; ++r) cf[r] *= G;
            for (int j0 = 0; j0 < h; j0 += 4) {
                const int jj = j0 + cg;
                const int jc = jj < h ? jj : 0;
                const float ej = jj < h ? s.ec[jc] : 0.f;
                float fx[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) fx[b] = ej * to_f<TR>(s.xc[(int64_t)jc * DV + 16 * (wv * NB + b) + rm]);
#pragma unroll
                for (int q = 0; q < NP; ++q) {
                    const float ka = to_f<TR>(s.kc[(int64_t)jc * DK + 16 * q + rm]);
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        cf[b * NP + q] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka, fx[b], cf[b * NP + q], 0, 0, 0);
                }
            }
            // plain stores (the two halves of a 128-byte line come from two
            // stores): 0-3 % faster per step than non-temporal ones here
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int q = 0; q < NP; ++q)
                    *reinterpret_cast<u32x4*>(ck + (int64_t)(16 * (wv * NB + b) + rm) * DK + 16 * q + 4 * cg) =
                        __builtin_bit_cast(u32x4, cf[b * NP + q]);
        }
    } else {
        // 4. outputs (each query scaled by its checkpoint weight first: T * VEC
        // multiplies instead of T * NR)
        float cf[NR][VEC];
        if (!TWO || fl) {
    #pragma unroll
            for (int r = 0; r < NR; ++r) unpack16<TS>(cb[r], cf[r]);
        } else {
    #pragma unroll
            for (int r = 0; r < NR; ++r) lq[r].to(cf[r], lsc[r]);
        }
        float acc[NV];
    #pragma unroll
        for (int i = 0; i < T; ++i) {
            const float g = s.gck[i ^ mq];
    #pragma unroll
            for (int c = 0; c < VEC; ++c) qv[i][c] *= g;
    #pragma unroll
            for (int r = 0; r < NR; ++r) {
                float a = 0.f;
    #pragma unroll
                for (int c = 0; c < VEC; ++c) a += cf[r][c] * qv[i][c];
                acc[i * NR + r] = a;
            }
        }
        for (int j = cc; j < nkeys; j += LPR) {
            float xj[NR];
    #pragma unroll
            for (int r = 0; r < NR; ++r)
                xj[r] = j < h ? to_f<TR>(s.xc[(int64_t)j * DV + r * RPP + rg]) : s.vd[(j - h) * DV + r * RPP + rg];
    #pragma unroll
            for (int i = 0; i < T; ++i) {
                const float wg = s.wq[j * T + (i ^ mq)];
    #pragma unroll
                for (int r = 0; r < NR; ++r) acc[i * NR + r] += wg * xj[r];
            }
        }
        xsum_perm<NV, LPR / 2, PL>(acc, cc);
        {
            constexpr int left = xsum_left<NV, LPR, 1>();
            if ((cc & xsum_dup_mask<NV, LPR, 1>()) == 0) {
                const int b0 = xsum_perm_base<NV, LPR, T>(cc);
    #pragma unroll
                for (int k = 0; k < left; ++k) {
                    const int v = b0 + k, i = v / NR, r = v - i * NR;
                    st_nt(p.out + ((tok0 + i) * p.n_heads + id.head) * DV + r * RPP + rg, acc[k]);
                }
            }
        }

        // 5. flush: fold the committed records (only those), store once
        if (fl) {  // uniform
            const float G = s.sc[1];
    #pragma unroll
            for (int r = 0; r < NR; ++r)
    #pragma unroll
                for (int c = 0; c < VEC; ++c) cf[r][c] *= G;
            for (int j = 0; j < h; ++j) {
                float kj[VEC];
                load_f<TR, VEC>(s.kc + (int64_t)j * DK + cc * VEC, kj);
                const float ej = s.ec[j];
    #pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const float f = ej * to_f<TR>(s.xc[(int64_t)j * DV + r * RPP + rg]);
    #pragma unroll
                    for (int c = 0; c < VEC; ++c) cf[r][c] += f * kj[c];
                }
            }
            bool stored = false;
            if constexpr (std::is_same<TS, tF16>::value) {
                if (p.sr) {
                    sr_store_rows<NR, 1, LPR>(cf, ck + (int64_t)rg * DK + cc * VEC, p, id.tile, rg, RPP, DK, cc * VEC);
                    stored = true;
                }
            }
            if (!stored) {
    #pragma unroll
                for (int r = 0; r < NR; ++r) st_stream(ck + (int64_t)(r * RPP + rg) * DK + cc * VEC, pack16<TS>(cf[r]));
            }
            if constexpr (TWO) {
    #pragma unroll
                for (int r = 0; r < NR; ++r)
                    store_read_quad<TL, LPR>(cf[r], cl + (int64_t)(r * RPP + rg) * DK + lpos, cs + r * RPP + rg, cc);
            }
        }
    }
    // drafts become records base .. base + T - 1 (keys: kbase .., the group's first head)
    if (key_owner) {
#pragma unroll
        for (int u = 0; u < QN; ++u) {
            const int e = (u * NT + tid) * 4;
            if (e < T * DK) {
                const int i = e / DK, c = e - i * DK;
                store_f<TR, 4>(rk + (int64_t)(kbase + i) * DK + c, s.kd + e);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < VN; ++u) {
        const int e = u * NT + tid;
        if (e < T * DV) {
            const int i = e / DV;
            st_nt(rx + (int64_t)(base + i) * DV + (e - i * DV), from_f<TR>(s.vd[e]));
        }
    }
    if (tid < T) st_nt(rl + base + tid, s.lamd[tid]);
}

// ---------------------------------- speculative verify, Gated DeltaNet form --
// A draft's corrected value u_i = beta_i (v_i - alpha_i S_{i-1} k_i) depends
// on the drafts before it (blog "The delta-rule wrinkle": a T x T triangular
// solve), so after the dot products the drafts are finished one at a time.
// With D_{a:b} the product of draft decays a..b and S_h the committed state
// (checkpoint plus committed records):
//   u_i = beta_i (v_i - D_{1:i} S_h k_i) - beta_i sum_{m<i} D_{m+1:i} (k_m . k_i) u_m
//   o_i = D_{1:i} S_h q_i + sum_{m<=i} D_{m+1:i} (k_m . q_i) u_m
// One workgroup per (row, head) tile (split 1, as k_spec_verify).
template <class R>
struct SpecGdnLds {
    R* kc;         // [slots][DK] committed keys
    R* xc;         // [DV][slots] committed corrected values, transposed so
                   // that lanes holding consecutive records read consecutive
                   // words (record-major would put a row group in one bank)
    float* qd;     // [T][DK] draft queries
    float* kd;     // [T][DK] draft keys
    float* vd;     // [T][DV] draft values
    float* lamd;   // [T] draft log-decays
    float* betad;  // [T] draft write strengths
    float* ec;     // [slots] exp(sum of the committed log-decays after record j)
    float* dexp;   // [T] D_{1:i}
    float* wdd;    // [T][T] D_{m+1:i} at [m * T + i], m <= i
    float* kq;     // [slots + T][T] key . q_i (committed keys, then drafts)
    float* kk;     // [slots + T][T] key . k_i
    float* sc;     // [4] total committed log-decay, its exponential
    float* y;      // [DV][spec_y_stride(T)] S_h q_i (columns i < T), S_h k_i
                   // (T + i): the matrix-core form only
};

// Row stride of SpecGdnLds::y: 2T products, 16-byte rows, 4 words of padding
// (the four lane groups of a wave write rows four apart).
constexpr int spec_y_stride(int T) { return (2 * T + 3) / 4 * 4 + 4; }

template <int DV, int DK, class R>
__device__ __forceinline__ SpecGdnLds<R> spec_gdn_carve(char* smem, int slots, int T) {
    SpecGdnLds<R> s;
    s.kc = reinterpret_cast<R*>(smem);
    s.xc = s.kc + (int64_t)slots * DK;
    float* f = reinterpret_cast<float*>(s.xc + (int64_t)slots * DV);
    s.qd = f;
    s.kd = s.qd + T * DK;
    s.vd = s.kd + T * DK;
    s.lamd = s.vd + T * DV;
    s.betad = s.lamd + T;
    s.ec = s.betad + T;
    s.dexp = s.ec + slots;
    s.wdd = s.dexp + T;
    s.kq = s.wdd + T * T;
    s.kk = s.kq + (slots + T) * T;
    s.sc = s.kk + (slots + T) * T;
    // 16-byte aligned, by arithmetic on the LDS pointer itself (a pointer
    // rebuilt from an integer is generic, and its loads wait like global ones)
    const size_t yoff = (size_t)(reinterpret_cast<char*>(s.sc + 4) - smem);
    s.y = reinterpret_cast<float*>(smem + ((yoff + 15) & ~size_t(15)));
    return s;
}

// The matrix-core form (spec_mf) adds the y rows and up to 12 bytes of
// alignment before them.
size_t spec_gdn_lds_bytes(int slots, int T, int dv, int dk, int rec_bytes, bool mf) {
    return (size_t)slots * (dk + dv) * rec_bytes +
           sizeof(float) * (2 * (size_t)T * dk + (size_t)T * dv + 2 * (size_t)T + (size_t)slots + (size_t)T +
                            (size_t)T * T + 2 * ((size_t)slots + T) * T + 4) +
           (mf ? 12 + sizeof(float) * (size_t)dv * spec_y_stride(T) : 0);
}


template <int DV, int DK, class TS, class TR, class TI, int T>
__global__ __launch_bounds__((Tile<DV, DK, TS, 1>::NT)) void k_spec_verify_gdn(const StepParams p) {
    using Tl = Tile<DV, DK, TS, 1>;
    constexpr bool MF = spec_mf(kGdn, DV, DK, std::is_same<TS, tF32>::value, T);
    using S = typename TS::S;
    using R = typename TR::S;
    using I = typename TI::S;
    constexpr int NT = Tl::NT, VEC = Tl::VEC, LPR = Tl::LPR, RPP = Tl::RPP, NR = Tl::NR;
    constexpr int QN = (T * DK / 4 + NT - 1) / NT;    // 4-element pieces of draft q / k per thread
    constexpr int VN = (T * DV + NT - 1) / NT;        // draft v elements per thread
    constexpr int KCH = DK * (int)sizeof(R) / 16, XCH = DV * (int)sizeof(R) / 16, XE = 16 / (int)sizeof(R);
    constexpr int RC = 2;                             // record chunks per thread in registers
    constexpr int NV = 2 * NR;                        // (S_h q_i, S_h k_i) partial sums of the owned rows
    static_assert(DK % 4 == 0 && VEC % 4 == 0, "4-element pieces");

    const TileIds id = tile_ids<1>(p);
    const uint8_t* fsrc = p.flush ? p.flush : reinterpret_cast<const uint8_t*>(p.write_pos);
    const bool flag = row_flag(fsrc, id.row) && p.flush;
    const int blk = p.block_table[id.row];
    const int h = p.write_pos[id.row];
    const bool pad = blk < 0;
    const bool bad = !pad && (blk >= p.n_blocks || h < 0 || h > p.slots);
    if (pad || bad) {
        if (bad) count_error(p, id);
        return;
    }
    const bool fl = flag || (h + T > p.L);  // no room for T more records: flush first
    const int base = fl ? 0 : h;            // slot of this step's first draft
    const int tid = threadIdx.x;
    const int cc = tid % LPR;
    const int rg = tid / LPR;
    // keys and queries per group (as k_spec_verify)
    const int grp = id.head / p.heads_per_group;
    const bool key_owner = id.head == grp * p.heads_per_group;
    const int kbase = fl && p.heads_per_group > 1 ? p.slots : base;

    char* bp = p.pool + (int64_t)blk * p.block_bytes;
    S* ck = reinterpret_cast<S*>(bp + p.ckpt_off) + (int64_t)id.head * (DV * DK);
    R* rx = reinterpret_cast<R*>(bp + p.recx_off) + (int64_t)id.head * p.slots * DV;
    R* rk = reinterpret_cast<R*>(bp + p.reck_off) + (int64_t)grp * p.key_slots * DK;
    float* rl = reinterpret_cast<float*>(bp + p.reclam_off) + (int64_t)id.head * p.slots;
    const I* qb = static_cast<const I*>(p.q) + id.row * p.qs_r + grp * p.qs_h;
    const I* kb = static_cast<const I*>(p.k) + id.row * p.ks_r + grp * p.ks_h;
    const I* vb = static_cast<const I*>(p.v) + id.row * p.vs_r + id.head * p.vs_h;
    const int64_t tok0 = (int64_t)id.row * T;

    extern __shared__ __attribute__((aligned(16))) char smem[];
    const SpecGdnLds<R> s = spec_gdn_carve<DV, DK, R>(smem, p.slots, T);

    // 1. small loads, then the checkpoint stream
    Raw4<TI> qr[QN], kr[QN];
#pragma unroll
    for (int u = 0; u < QN; ++u) {
        const int e = min((u * NT + tid) * 4, T * DK - 4);  // clamped: every thread loads
        const int i = e / DK, c = e - i * DK;
        qr[u].load(qb + i * p.qs_t + c);
        kr[u].load(kb + i * p.ks_t + c);
    }
    I vr[VN];
#pragma unroll
    for (int u = 0; u < VN; ++u) {
        const int e = min(u * NT + tid, T * DV - 1);
        const int i = e / DV;
        vr[u] = vb[i * p.vs_t + (e - i * DV)];
    }
    const int64_t dtok = (tok0 + min(tid, T - 1)) * p.n_heads + id.head;
    const float lam_d = p.lam[dtok];
    const float beta_d = p.beta[dtok];
    float lam_c = 0.f;
    if (h > 0) lam_c = rl[min(tid, h - 1)];
    const int nk = h * KCH, nrec = nk + h * XCH;
    auto rsrc = [&](int i) -> const R* {
        if (i < nk) return rk + (int64_t)i * XE;
        const int t2 = i - nk, j = t2 / XCH;
        return rx + (int64_t)j * DV + (t2 - j * XCH) * XE;
    };
    auto put = [&](int i, u32x4 v) {  // keys as chunks, corrected values transposed
        if (i < nk) {
            reinterpret_cast<u32x4*>(s.kc)[i] = v;
            return;
        }
        const int t2 = i - nk, j = t2 / XCH, e0 = (t2 - j * XCH) * XE;
        R e[XE];
        __builtin_memcpy(e, &v, 16);
#pragma unroll
        for (int x = 0; x < XE; ++x) s.xc[(e0 + x) * p.slots + j] = e[x];
    };
    u32x4 rb[RC];
    if (nrec > 0) {
#pragma unroll
        for (int u = 0; u < RC; ++u) rb[u] = ld_stream(rsrc(min(u * NT + tid, nrec - 1)));
    }
    for (int i = RC * NT + tid; i < nrec; i += NT) put(i, ld_stream(rsrc(i)));
    // Matrix-core form: wave wv owns the 16-row blocks wv NB .. wv NB + NB - 1;
    // in block b, lane (rm, cg) holds row 16 (wv NB + b) + rm, columns
    // 16 q + 4 cg .. + 3 of every 16-column slice q (one 64-byte piece of 16
    // rows per load).  That is the A operand of the 16 x 16 x 4 fp32 matrix
    // product, one column per lane group, so S_h [q, k] needs no exchange.
    // Plain loads: the two halves of a 128-byte line come from two loads,
    // and non-temporal ones measured 2-5 % slower here.
    constexpr int NB = DV / 64, NP = DK / 16;
    [[maybe_unused]] const int wv = tid >> 6, rm = tid & 15, cg = (tid >> 4) & 3;
    u32x4 cb[NR];
    if constexpr (MF) {
        static_assert(NB * NP == NR && NT == 256, "four waves of 16-row blocks");
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int q = 0; q < NP; ++q)
                cb[b * NP + q] = *reinterpret_cast<const u32x4*>(ck + (int64_t)(16 * (wv * NB + b) + rm) * DK + 16 * q + 4 * cg);
    } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) cb[r] = ld_stream(ck + (int64_t)(r * RPP + rg) * DK + cc * VEC);
    }

    // 2. to LDS
#pragma unroll
    for (int u = 0; u < QN; ++u) {
        const int e = (u * NT + tid) * 4;
        if (e < T * DK) {
            qr[u].to(s.qd + e);
            kr[u].to(s.kd + e);
        }
    }
#pragma unroll
    for (int u = 0; u < VN; ++u)
        if (u * NT + tid < T * DV) s.vd[u * NT + tid] = to_f<TI>(vr[u]);
    if (tid < T) {
        s.lamd[tid] = lam_d;
        s.betad[tid] = beta_d;
    }
#pragma unroll
    for (int u = 0; u < RC; ++u)
        if (u * NT + tid < nrec) put(u * NT + tid, rb[u]);
    __syncthreads();

    // 3. decay weights (wave 0)
    if (tid < 64) {
        const int lane = tid;
        float sfx = lane < h ? lam_c : 0.f;  // inclusive suffix sum of the committed log-decays
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float t = __shfl_down(sfx, off);
            if (lane + off < 64) sfx += t;
        }
        float after = __shfl_down(sfx, 1);
        if (lane == 63) after = 0.f;
        if (lane < h) s.ec[lane] = expf(after);
        if (lane == 0) {
            s.sc[0] = sfx;
            s.sc[1] = expf(sfx);
        }
        if (lane < T) {  // D_{1:i} and D_{m+1:i} from the draft log-decays
            float c = 0.f;
            for (int m = 0; m <= lane; ++m) c += s.lamd[m];
            s.dexp[lane] = expf(c);
            for (int m = 0; m <= lane; ++m) {
                float sm = 0.f;
                for (int l = m + 1; l <= lane; ++l) sm += s.lamd[l];
                s.wdd[m * T + lane] = expf(sm);
            }
        }
    }

    // 4. every key (committed, then draft) against every draft's q and k
    const int nkeys = h + T;
    for (int j0 = 0; j0 < nkeys; j0 += RPP) {
        const int j = j0 + rg;
        float kj[VEC];
        if (j < h) {
            load_f<TR, VEC>(s.kc + (int64_t)j * DK + cc * VEC, kj);
        } else {
            const int m = min(j - h, T - 1);
#pragma unroll
            for (int c = 0; c < VEC; ++c) kj[c] = s.kd[m * DK + cc * VEC + c];
        }
        float part[2 * T];
#pragma unroll
        for (int i = 0; i < T; ++i) {
            float a = 0.f, b = 0.f;
#pragma unroll
            for (int c = 0; c < VEC; ++c) {
                a += kj[c] * s.qd[i * DK + cc * VEC + c];
                b += kj[c] * s.kd[i * DK + cc * VEC + c];
            }
            part[i] = a;
            part[T + i] = b;
        }
        xsum<2 * T, LPR / 2, 1>(part, cc);
        constexpr int left = xsum_left<2 * T, LPR, 1>();
        if (j < nkeys && (cc & xsum_dup_mask<2 * T, LPR, 1>()) == 0) {
            const int b0 = xsum_base<2 * T, LPR, 1>(cc);
#pragma unroll
            for (int x = 0; x < left; ++x) {
                const int v = b0 + x;
                if (v < T) s.kq[j * T + v] = part[x];
                else s.kk[j * T + v - T] = part[x];
            }
        }
    }
    __syncthreads();

    if constexpr (MF) {
        using f4 = __attribute__((ext_vector_type(4))) float;
        constexpr int YS = spec_y_stride(T);
        const float P = s.sc[1];
        f4 cf[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) cf[r] = __builtin_bit_cast(f4, cb[r]);
        // 5. Y = P S_h W + X G on the matrix cores, W = [q_1 .. q_T, k_1 .. k_T]
        //    (d_k x 2T, zero beyond), X the committed corrected values, G_jn =
        //    e_j (k_j . w_n).  Each 16 x 16 x 4 product takes four columns of
        //    16 rows (lane group cg holds column 4 cg + e of slice q) against
        //    the same columns of W (lane (rm, cg): column n = rm); lane (rm, cg)
        //    ends with rows 4 cg .. + 3 of the block at column n = rm.
        const int nq = min(rm, T - 1), nkd = min(max(rm - T, 0), T - 1);
        const float* wsrc = (rm < T ? s.qd + nq * DK : s.kd + nkd * DK) + 4 * cg;
        const float wsc = rm < 2 * T ? P : 0.f;
        f4 y[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) y[b] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const f4 w = *reinterpret_cast<const f4*>(wsrc + 16 * q) * wsc;
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int b = 0; b < NB; ++b) y[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(cf[b * NP + q][e], w[e], y[b], 0, 0, 0);
        }
        // records four at a time; a slot past h takes slot 0's (finite) value
        // with weight zero
        for (int j0 = 0; j0 < h; j0 += 4) {
            const int jj = j0 + cg;
            const int jc = jj < h ? jj : 0;
            const float g = jj < h && rm < 2 * T ? s.ec[jc] * (rm < T ? s.kq[jc * T + nq] : s.kk[jc * T + nkd]) : 0.f;
#pragma unroll
            for (int b = 0; b < NB; ++b)
                y[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(to_f<TR>(s.xc[(16 * (wv * NB + b) + rm) * p.slots + jc]), g,
                                                            y[b], 0, 0, 0);
        }
        if (rm < 2 * T) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) s.y[(16 * (wv * NB + b) + 4 * cg + i) * YS + rm] = y[b][i];
        }
        // 6. flush (before the substitution, so that the tile's registers are
        //    free there): S_h = P C + sum_j e_j x_j k_j^T on the matrix cores, in
        //    place: as C^T += K^T F^T a lane's four values of slice q are rows
        //    4 cg .. + 3 of the product at column rm, A = keys (slot j0 + cg,
        //    column 16 q + rm), B = F (row rm of the block, slot j0 + cg)
        if (fl) {  // uniform
#pragma unroll
            for (int r = 0; r < NR; ++r) cf[r] *= P;
            for (int j0 = 0; j0 < h; j0 += 4) {
                const int jj = j0 + cg;
                const int jc = jj < h ? jj : 0;
                const float ej = jj < h ? s.ec[jc] : 0.f;
                float fx[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) fx[b] = ej * to_f<TR>(s.xc[(16 * (wv * NB + b) + rm) * p.slots + jc]);
#pragma unroll
                for (int q = 0; q < NP; ++q) {
                    const float ka = to_f<TR>(s.kc[(int64_t)jc * DK + 16 * q + rm]);
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        cf[b * NP + q] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka, fx[b], cf[b * NP + q], 0, 0, 0);
                }
            }
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int q = 0; q < NP; ++q)
                    st_stream(ck + (int64_t)(16 * (wv * NB + b) + rm) * DK + 16 * q + 4 * cg,
                              __builtin_bit_cast(u32x4, cf[b * NP + q]));
        }
        __syncthreads();
        // substitution, one thread per state row; outputs and the drafts'
        // corrected values (records base .. base + T - 1)
        if (tid < DV) {
            const int row = tid;
            float yv[2 * T];
#pragma unroll
            for (int n = 0; n < 2 * T; ++n) yv[n] = s.y[row * YS + n];
            float ur[T];
#pragma unroll
            for (int i = 0; i < T; ++i) {
                const float D = s.dexp[i], bt = s.betad[i];
                float u = bt * (s.vd[i * DV + row] - D * yv[T + i]);
                float o = D * yv[i];
#pragma unroll
                for (int m = 0; m < i; ++m) {
                    const float w = s.wdd[m * T + i];
                    u -= bt * w * s.kk[(h + m) * T + i] * ur[m];
                    o += w * s.kq[(h + m) * T + i] * ur[m];
                }
                o += s.kq[(h + i) * T + i] * u;  // m = i, weight 1
                ur[i] = u;
                st_nt<kNtSmall<kGdn>>(p.out + ((tok0 + i) * p.n_heads + id.head) * DV + row, o);
                st_nt<kNtSmall<kGdn>>(rx + (int64_t)(base + i) * DV + row, from_f<TR>(u));
            }
        }
        // 7. the drafts' keys (kbase .., the group's first head)
        if (key_owner) {
#pragma unroll
            for (int u = 0; u < QN; ++u) {
                const int e = (u * NT + tid) * 4;
                if (e < T * DK) {
                    const int i = e / DK, c = e - i * DK;
                    store_f<TR, 4, kNtSmall<kGdn>>(rk + (int64_t)(kbase + i) * DK + c, s.kd + e);
                }
            }
        }
    } else {
        // 5. drafts in order: S_h q_i, S_h k_i for the owned rows, then the
        //    substitution and the output at the lanes that own each row
        float cf[NR][VEC];
    #pragma unroll
        for (int r = 0; r < NR; ++r) unpack16<TS>(cb[r], cf[r]);
        const float P = s.sc[1];
        constexpr int left = xsum_left<NV, LPR, 2>();
        constexpr int NOWN = left / 2;  // rows this lane ends up with
        const int b0 = xsum_base<NV, LPR, 2>(cc);
        const bool owner = (cc & xsum_dup_mask<NV, LPR, 2>()) == 0;
        float ur[T][NOWN];  // corrected values of the owned rows, drafts so far
    #pragma unroll
        for (int i = 0; i < T; ++i) {
            float acc[NV];
    #pragma unroll
            for (int r = 0; r < NR; ++r) {
                float a = 0.f, b = 0.f;
    #pragma unroll
                for (int c = 0; c < VEC; ++c) {
                    a += cf[r][c] * s.qd[i * DK + cc * VEC + c];
                    b += cf[r][c] * s.kd[i * DK + cc * VEC + c];
                }
                acc[2 * r] = P * a;
                acc[2 * r + 1] = P * b;
            }
            for (int j = cc; j < h; j += LPR) {
                const float wq = s.ec[j] * s.kq[j * T + i], wk = s.ec[j] * s.kk[j * T + i];
    #pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const float u = to_f<TR>(s.xc[(r * RPP + rg) * p.slots + j]);
                    acc[2 * r] += wq * u;
                    acc[2 * r + 1] += wk * u;
                }
            }
            xsum<NV, LPR / 2, 2>(acc, cc);
            const float D = s.dexp[i], bt = s.betad[i];
    #pragma unroll
            for (int x = 0; x < NOWN; ++x) {
                const int row = ((b0 + 2 * x) / 2) * RPP + rg;
                float u = bt * (s.vd[i * DV + row] - D * acc[2 * x + 1]);
                float o = D * acc[2 * x];
    #pragma unroll
                for (int m = 0; m < i; ++m) {
                    const float w = s.wdd[m * T + i];
                    u -= bt * w * s.kk[(h + m) * T + i] * ur[m][x];
                    o += w * s.kq[(h + m) * T + i] * ur[m][x];
                }
                o += s.kq[(h + i) * T + i] * u;  // m = i, weight 1
                ur[i][x] = u;
                if (owner) st_nt<kNtSmall<kGdn>>(p.out + ((tok0 + i) * p.n_heads + id.head) * DV + row, o);
            }
        }

        // 6. flush: fold the committed records (only those), store once
        if (fl) {  // uniform
    #pragma unroll
            for (int r = 0; r < NR; ++r)
    #pragma unroll
                for (int c = 0; c < VEC; ++c) cf[r][c] *= P;
            for (int j = 0; j < h; ++j) {
                float kj[VEC];
                load_f<TR, VEC>(s.kc + (int64_t)j * DK + cc * VEC, kj);
                const float ej = s.ec[j];
    #pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const float f = ej * to_f<TR>(s.xc[(r * RPP + rg) * p.slots + j]);
    #pragma unroll
                    for (int c = 0; c < VEC; ++c) cf[r][c] += f * kj[c];
                }
            }
            bool stored = false;
            if constexpr (std::is_same<TS, tF16>::value) {
                if (p.sr) {
                    sr_store_rows<NR, 1, LPR>(cf, ck + (int64_t)rg * DK + cc * VEC, p, id.tile, rg, RPP, DK, cc * VEC);
                    stored = true;
                }
            }
            if (!stored) {
    #pragma unroll
                for (int r = 0; r < NR; ++r) st_stream(ck + (int64_t)(r * RPP + rg) * DK + cc * VEC, pack16<TS>(cf[r]));
            }
        }
        // 7. drafts become records base .. base + T - 1: keys (kbase .., the
        // group's first head), corrected values, log-decays
        if (key_owner) {
    #pragma unroll
            for (int u = 0; u < QN; ++u) {
                const int e = (u * NT + tid) * 4;
                if (e < T * DK) {
                    const int i = e / DK, c = e - i * DK;
                    store_f<TR, 4, kNtSmall<kGdn>>(rk + (int64_t)(kbase + i) * DK + c, s.kd + e);
                }
            }
        }
        if (owner) {
    #pragma unroll
            for (int i = 0; i < T; ++i)
    #pragma unroll
                for (int x = 0; x < NOWN; ++x)
                    st_nt<kNtSmall<kGdn>>(rx + (int64_t)(base + i) * DV + ((b0 + 2 * x) / 2) * RPP + rg, from_f<TR>(ur[i][x]));
        }
    }
    if (tid < T) st_nt<kNtSmall<kGdn>>(rl + base + tid, s.lamd[tid]);
}

// Grouped keys: a row that flushed in its verify has its drafts' keys in the
// staging slots (slots .. slots + T - 1 of each group); move the accepted
// ones to slots 0 .. a - 1.  One workgroup per (row, group), 16-byte chunks.
// Reads the same metadata as k_spec_commit, which writes other arrays.
__global__ __launch_bounds__(64) void k_spec_commit_keys(const StepParams p) {
    const int row = blockIdx.y, grp = blockIdx.x;
    const int blk = p.block_table[row];
    if (blk < 0) return;
    const int h = p.write_pos[row];
    const int T = p.spec_T;
    if (blk >= p.n_blocks || h < 0 || h > p.slots) return;  // counted by k_spec_commit
    const bool fl = (p.flush && p.flush[row]) || (h + T > p.L);
    const int a = p.accepted[row];
    if (!fl || a < 1 || a > T) return;
    char* keys = p.pool + (int64_t)blk * p.block_bytes + p.reck_off + (int64_t)grp * p.key_slots * p.key_bytes;
    const int n = a * p.key_bytes / 16;  // key_bytes is a multiple of 16
    const u32x4* src = reinterpret_cast<const u32x4*>(keys + (int64_t)p.slots * p.key_bytes);
    u32x4* dst = reinterpret_cast<u32x4*>(keys);
    for (int i = threadIdx.x; i < n; i += 64) dst[i] = src[i];
}

// Commit after a verify: one thread per row (see replay_spec_commit).
__global__ __launch_bounds__(256) void k_spec_commit(const StepParams p) {
    const int row = blockIdx.x * 256 + threadIdx.x;
    if (row >= p.n_rows) return;
    const int blk = p.block_table[row];
    if (blk < 0) return;
    const int h = p.write_pos[row];
    const int T = p.spec_T;
    if (blk >= p.n_blocks || h < 0 || h > p.slots) {
        if (p.err) atomicAdd(p.err, 1);
        return;
    }
    const bool fl = (p.flush && p.flush[row]) || (h + T > p.L);
    int a = p.accepted[row];
    if (a < 0 || a > T) {
        if (p.err) atomicAdd(p.err, 1);
        a = 0;
    }
    const int hn = (fl ? 0 : h) + a;
    p.next_wp[row] = hn;
    p.next_flush[row] = (uint8_t)(hn + T > p.L ? 1 : 0);
}

// ------------------------------------------------------------ state reset --
// Zero the checkpoint (both copies of a two-precision checkpoint).
template <int DV, int DK, class TS, int SPLIT, class TL>
__global__ __launch_bounds__((Tile<DV, DK, TS, SPLIT>::NT)) void k_state_reset(const StepParams p) {
    using T = Tile<DV, DK, TS, SPLIT>;
    using S = typename TS::S;
    using RL = typename TL::S;
    constexpr int NT = T::NT, NR = T::NR, DVW = T::DVW;
    constexpr bool TWO = !std::is_same<TS, TL>::value;
    const TileIds id = tile_ids<SPLIT>(p);
    const bool m = row_flag(p.mask, id.row);
    const int blk = p.block_table[id.row];
    if (blk < 0 || !m) return;
    if (blk >= p.n_blocks) {
        count_error(p, id);
        return;
    }
    char* base = p.pool + (int64_t)blk * p.block_bytes;
    const int64_t elem0 = (int64_t)id.head * (DV * DK) + (int64_t)id.part * DVW * DK;
    S* ck = reinterpret_cast<S*>(base + p.ckpt_off) + elem0;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < NR; ++r) st_stream(reinterpret_cast<u32x4*>(ck) + r * NT + threadIdx.x, z);
    if constexpr (TWO) {
        // the read copy's owned rows are DVW * DK * sizeof(RL) bytes
        constexpr int CH = DVW * DK * (int)sizeof(RL) / 16;
        RL* cl = reinterpret_cast<RL*>(base + p.ckpt_lo_off) + elem0;
        for (int i = threadIdx.x; i < CH; i += NT) st_stream(reinterpret_cast<u32x4*>(cl) + i, z);
        if constexpr (kScaled<TL>) {
            float* cs = reinterpret_cast<float*>(base + p.ckpt_sc_off) + id.head * DV + id.part * DVW;
            if ((int)threadIdx.x < DVW) cs[threadIdx.x] = 0.f;
        }
    }
}

// How many workgroups share one (row, head) tile: at most 8192 state elements
// (32 floats per thread at 256 threads) per workgroup.  Measured on MI355X:
// with more, the extra registers cost occupancy (Gated DeltaNet's fp16 128x128
// tile: 5.2 TB/s unsplit, 5.8 TB/s split in two); below it, splitting further
// only repeats the record dot products.
template <int DV, int DK>
constexpr int split_for() {
    constexpr int s = DV * DK / 8192;
    return s < 1 ? 1 : s;
}

// The replay step's split for a single checkpoint: whole tiles up to 32 KiB
// of state per workgroup.  Measured on MI355X, Gated DeltaNet 128 x 128 with
// an fp16 state, batch 256: window average 64.6 -> 58.7 us per launch
// unsplit (fp32 state, 64 KiB per tile, keeps split_for).  The read-modify-
// write kernels keep split_for: the conventional step measured 5 % slower
// unsplit (90.1 -> 95.2 us).
template <int DV, int DK, class TS>
constexpr int replay_split() {
    return DV * DK * (int)sizeof(typename TS::S) <= 32768 ? 1 : split_for<DV, DK>();
}

// Whether Tile<DV, DK, TS, SPLIT> is a valid decomposition (the conditions
// its static_asserts check, plus at least 8 owned rows so that an owned value
// record is a whole number of 16-byte chunks).
template <int DV, int DK, class TS, int SPLIT>
constexpr bool tile_ok() {
    if (SPLIT < 1 || DV % SPLIT) return false;
    const int dvw = DV / SPLIT;
    const int vec = 16 / (int)sizeof(typename TS::S);
    const int lpr = DK / vec;
    const int loads = dvw * lpr;
    const int per = kScaled<TS> ? 2 : 4;
    const int nt = loads / per >= 256 ? 256 : (loads / per >= 128 ? 128 : 64);
    if (lpr < 1 || lpr > 64 || (lpr & (lpr - 1)) || nt % lpr) return false;
    const int rpp = nt / lpr;
    if (dvw % rpp) return false;
    const int nr = dvw / rpp;
    return nr >= 1 && (nr & (nr - 1)) == 0 && nt >= dvw && dvw >= 8;
}

// A wider split for grids too small to fill the chip: up to 8x the base.
template <int DV, int DK, class TS>
constexpr int wide_split() {
    constexpr int b = split_for<DV, DK>();
    if constexpr (tile_ok<DV, DK, TS, 8 * b>()) return 8 * b;
    else if constexpr (tile_ok<DV, DK, TS, 4 * b>()) return 4 * b;
    else if constexpr (tile_ok<DV, DK, TS, 2 * b>()) return 2 * b;
    else return b;
}

// Read-modify-write launches (conventional step, token-less flush) with fewer
// workgroups than this (4 per compute unit) use the wide split: a small batch
// is bound by each workgroup's latency, not by bandwidth.
constexpr int64_t kFillWorkgroups = 1024;

// -------------------------------------------------------------- dispatch --
// Persistent launch shape of a replay step: the grid (0: launch the
// one-workgroup-per-tile form instead), where the deferred writes start in
// LDS, how many tiles they hold, and the LDS size.
struct PersistShape {
    unsigned grid = 0;
    int meta_off = 0, defer_off = 0, defer_cap = 0;
    size_t lds = 0;
};
constexpr int kMaxDefer = 64;
// Workgroups per compute unit (measured on MI355X, Nemotron-3-Super shape,
// batch 256: 2 beat 3 and 4; fewer workgroups also make the deferred writes'
// end-of-launch burst shorter).
constexpr int kPersistPerCU = 2;

// Workgroups of fn (nt threads, lds bytes) resident per compute unit, cached
// per device (the occupancy query reads the kernel's register counts).
int resident_per_cu(const void* fn, int nt, size_t lds, int dev) {
    struct Entry {
        const void* fn;
        size_t lds;
        int dev, nb;
    };
    static std::mutex m;
    static std::vector<Entry> cache;
    std::lock_guard<std::mutex> g(m);
    for (const Entry& e : cache)
        if (e.fn == fn && e.lds == lds && e.dev == dev) return e.nb;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, nt, lds) != hipSuccess) nb = 0;
    cache.push_back({fn, lds, dev, nb});
    return nb;
}

// lds0: the records area of one item; the persistent step keeps two.
PersistShape persist_shape(const void* fn, int nt, size_t lds0, int entry_bytes, int64_t items) {
    PersistShape r;
    int dev = 0, cus = 0, lds_cu = 0;
    if (items < 1 || hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
        cus < 1)
        return r;
    const int off = 2 * (int)((lds0 + 15) / 16 * 16);
    const int per_cu = std::min(kPersistPerCU, resident_per_cu(fn, nt, (size_t)off, dev));
    if (per_cu < 1) return r;
    const int64_t grid = std::min<int64_t>(items, (int64_t)per_cu * cus);
    const int64_t mine = (items + grid - 1) / grid;  // most items of one workgroup
    const int64_t meta = 32 + (mine * 12 + 15) / 16 * 16;  // counters, then 3 ints per running item
    const int64_t room = (int64_t)lds_cu / per_cu - off - meta;
    const int64_t cap = std::min<int64_t>({room / entry_bytes, mine, kMaxDefer});
    if (cap < 1) return r;
    const size_t lds = (size_t)(off + meta + cap * entry_bytes);
    if (resident_per_cu(fn, nt, lds, dev) < per_cu) return r;
    r.grid = (unsigned)grid;
    r.meta_off = off;
    r.defer_off = (int)(off + meta);
    r.defer_cap = (int)cap;
    r.lds = lds;
    return r;
}

template <int DV, int DK, class TS, class F>
void with_split(const StepParams* p, F&& f) {
    constexpr int base = split_for<DV, DK>();
    constexpr int wide = wide_split<DV, DK, TS>();
    if constexpr (wide != base) {
        if (p && (int64_t)p->n_rows * p->n_heads * base < kFillWorkgroups) {
            f(std::integral_constant<int, wide>{});
            return;
        }
    }
    f(std::integral_constant<int, base>{});
}

template <class F>
bool with_state(int dt, F&& f) {
    if (dt == RS_F32) { f(tF32{}); return true; }
    if (dt == RS_F16) { f(tF16{}); return true; }
    return false;
}
template <class F>
bool with_record(int dt, F&& f) { return with_state(dt, f); }
template <class F>
bool with_io(int dt, F&& f) {
    if (dt == RS_BF16) { f(tBF16{}); return true; }
    return with_state(dt, f);
}
template <class F>
bool with_shape(int dv, int dk, F&& f) {
    if (dv == 16 && dk == 32) { f(std::integral_constant<int, 16>{}, std::integral_constant<int, 32>{}); return true; }
    if (dv == 64 && dk == 128) { f(std::integral_constant<int, 64>{}, std::integral_constant<int, 128>{}); return true; }
    if (dv == 128 && dk == 128) { f(std::integral_constant<int, 128>{}, std::integral_constant<int, 128>{}); return true; }
    return false;
}
template <class F>
bool with_spec_T(int T, F&& f) {
    if (T == 1) { f(std::integral_constant<int, 1>{}); return true; }
    if (T == 2) { f(std::integral_constant<int, 2>{}); return true; }
    if (T == 4) { f(std::integral_constant<int, 4>{}); return true; }
    if (T == 8) { f(std::integral_constant<int, 8>{}); return true; }
    return false;
}
template <class F>
bool with_form(int form, F&& f) {
    if (form == RS_MAMBA2) { f(std::integral_constant<int, kMamba2>{}); return true; }
    if (form == RS_GDN) { f(std::integral_constant<int, kGdn>{}); return true; }
    return false;
}

// The read copy's type: the state type itself (one checkpoint), or, for a
// two-precision checkpoint, fp16 / bf16 / E4M3 over an fp32 recurrence copy
// and E4M3 over an fp16 one.  E4M3 needs a head of at least one wave of
// 16-byte code chunks (64 x 128 and 128 x 128; not 16 x 32).
template <int DV, int DK, class TS, class F>
bool with_read(int read_dt, int state_dt, F&& f) {
    if (read_dt < 0 || read_dt == state_dt) { f(TS{}); return true; }
    if constexpr (std::is_same<TS, tF32>::value) {
        if (read_dt == RS_F16) { f(tF16{}); return true; }
        if (read_dt == RS_BF16) { f(tBF16{}); return true; }
    }
    if constexpr (std::is_same<TS, tF32>::value || std::is_same<TS, tF16>::value) {
        if constexpr (tile_ok<DV, DK, tE4M3, split_for<DV, DK>()>()) {
            if (read_dt == RS_E4M3) { f(tE4M3{}); return true; }
        }
    }
    return false;
}

struct Dispatch {
    Kind kind;
    const rs_layer& L;
    const StepParams* p;   // nullptr: only check that a kernel exists
    hipStream_t stream;
    hipError_t err = hipSuccess;

    template <int SPLIT>
    dim3 grid() const {
        return dim3(p ? (unsigned)(p->n_heads * SPLIT) : 1u, p ? (unsigned)p->n_rows : 1u);
    }

    bool run() {
        // record slots per head: the block layout's (a speculative ring holds
        // L committed records, a standard buffer L - 1)
        const int slots = L.spec_T > 0 ? L.L : L.L - 1;
        bool ok = false;
        with_shape(L.d_v, L.d_k, [&](auto dv_c, auto dk_c) {
            constexpr int DV = decltype(dv_c)::value, DK = decltype(dk_c)::value;
            with_state(L.state_dtype, [&](auto ts) {
                using TS = decltype(ts);
                if (kind == Kind::ConventionalStep) {
                    with_form(L.form, [&](auto f_c) {
                        constexpr int FORM = decltype(f_c)::value;
                        with_io(L.io_dtype, [&](auto ti) {
                            using TI = decltype(ti);
                            ok = true;
                            if (p)
                                with_split<DV, DK, TS>(p, [&](auto sp_c) {
                                    constexpr int SP = decltype(sp_c)::value;
                                    hipLaunchKernelGGL((k_conventional_step<FORM, DV, DK, TS, TI, SP>), grid<SP>(),
                                                       dim3(Tile<DV, DK, TS, SP>::NT), 0, stream, *p);
                                });
                        });
                    });
                    return;
                }
                if (kind == Kind::SpecVerify) {
                    with_form(L.form, [&](auto f_c) {
                        constexpr int FORM = decltype(f_c)::value;
                        // one workgroup per (row, head) tile, 128 x 128 included
                        constexpr bool have = tile_ok<DV, DK, TS, 1>();
                        if constexpr (have) {
                            with_record(L.record_dtype, [&](auto tr) {
                                using TR = decltype(tr);
                                with_io(L.io_dtype, [&](auto ti) {
                                    using TI = decltype(ti);
                                    with_spec_T(L.spec_T, [&](auto t_c) {
                                        constexpr int T = decltype(t_c)::value;
                                        const int rb = (int)sizeof(typename TR::S);
                                        const dim3 block(Tile<DV, DK, TS, 1>::NT);
                                        if constexpr (FORM == kMamba2) {
                                            // a read copy only under an fp32 recurrence copy
                                            with_read<DV, DK, TS>(L.read_dtype, L.state_dtype, [&](auto tl) {
                                                using TL = decltype(tl);
                                                if constexpr (std::is_same<TS, TL>::value ||
                                                              std::is_same<TS, tF32>::value) {
                                                    ok = true;
                                                    if (!p) return;
                                                    hipLaunchKernelGGL((k_spec_verify<DV, DK, TS, TR, TI, T, TL>), grid<1>(),
                                                                       block, spec_lds_bytes(L.L, T, DV, DK, rb), stream,
                                                                       *p);
                                                }
                                            });
                                        } else if (L.read_dtype < 0 || L.read_dtype == L.state_dtype) {
                                            ok = true;
                                            if (!p) return;
                                            hipLaunchKernelGGL((k_spec_verify_gdn<DV, DK, TS, TR, TI, T>), grid<1>(),
                                                               block,
                                                               spec_gdn_lds_bytes(L.L, T, DV, DK, rb,
                                                                                  spec_mf(kGdn, DV, DK, std::is_same<TS, tF32>::value, T)),
                                                               stream,
                                                               *p);
                                        }
                                    });
                                });
                            });
                        }
                    });
                    return;
                }
                if (kind == Kind::SpecCommit) {
                    ok = true;
                    if (p && p->heads_per_group > 1)
                        hipLaunchKernelGGL(k_spec_commit_keys, dim3((unsigned)(p->n_heads / p->heads_per_group),
                                                                    (unsigned)p->n_rows),
                                           dim3(64), 0, stream, *p);
                    if (p)
                        hipLaunchKernelGGL(k_spec_commit, dim3((unsigned)((p->n_rows + 255) / 256)), dim3(256), 0,
                                           stream, *p);
                    return;
                }
                with_read<DV, DK, TS>(L.read_dtype, L.state_dtype, [&](auto tl) {
                    using TL = decltype(tl);
                    constexpr bool TWO = !std::is_same<TS, TL>::value;
                    if (kind == Kind::Reset) {
                        constexpr int SP = split_for<DV, DK>();
                        ok = true;
                        if (p)
                            hipLaunchKernelGGL((k_state_reset<DV, DK, TS, SP, TL>), grid<SP>(),
                                               dim3(Tile<DV, DK, TS, SP>::NT), 0, stream, *p);
                        return;
                    }
                    with_record(L.record_dtype, [&](auto tr) {
                        using TR = decltype(tr);
                        using R = typename TR::S;
                        if (kind == Kind::Flush) {
                            ok = true;
                            if (p)
                                with_split<DV, DK, TL>(p, [&](auto sp_c) {
                                    constexpr int SP = decltype(sp_c)::value;
                                    const size_t lds = lds_need<DV / SP, DK, R>(slots, L.L);
                                    hipLaunchKernelGGL((k_replay_flush<DV, DK, TS, TR, SP, TL>), grid<SP>(),
                                                       dim3(Tile<DV, DK, TL, SP>::NT), lds, stream, *p);
                                });
                            return;
                        }
                        with_form(L.form, [&](auto f_c) {
                            constexpr int FORM = decltype(f_c)::value;
                            if constexpr (TWO && FORM != kMamba2) {
                                return;  // two-precision checkpoint: Mamba-2 form only
                            } else {
                                with_io(L.io_dtype, [&](auto ti) {
                                    using TI = decltype(ti);
                                    ok = true;
                                    if (p) {
                                        // Unsplit tiles of up to 32 KiB (replay_split) when the
                                        // grid fills the chip, else split_for; never wider:
                                        // measured, a wider split at small batch repeats the
                                        // record work in more workgroups and is slower
                                        // (Gated DeltaNet batch 1: 9.1 -> 10.3 us).
                                        constexpr int SPW = TWO ? split_for<DV, DK>() : replay_split<DV, DK, TS>();
                                        constexpr int SPB = split_for<DV, DK>();
                                        const bool whole = (int64_t)p->n_rows * p->n_heads >= kFillWorkgroups;
                                        auto go = [&](auto sp_c) {
                                            constexpr int SP = decltype(sp_c)::value;
                                            const size_t lds = lds_need<DV / SP, DK, R>(slots, L.L);
                                            const dim3 block(Tile<DV, DK, TL, SP>::NT);
                                            if constexpr (FORM == kGdn) {
                                                if (p->reconstruct) {  // (the hint is cleared for it)
                                                    hipLaunchKernelGGL((k_replay_step<FORM, DV, DK, TS, TR, TI, SP, TL, true>),
                                                                       grid<SP>(), block, lds, stream, *p);
                                                    return;
                                                }
                                            }
                                            const int hint = p->flush_hint;
                                            // The persistent form (steps with no flushing row)
                                            // for Mamba-2 with one fp32 checkpoint and a key per
                                            // head, where it measured faster; with 16-bit tiles,
                                            // read copies or Gated DeltaNet two workgroups per
                                            // compute unit keep too little in flight, and with
                                            // grouped keys (a key append in one tile of a group)
                                            // there is less interleaved writing to take out: it
                                            // measured slower there.
                                            constexpr bool persist_form =
                                                FORM == kMamba2 && !TWO && std::is_same<TS, tF32>::value;
                                            if constexpr (persist_form) {
                                                if (hint == RS_FLUSH_NONE && p->heads_per_group == 1) {
                                                    // It copies the records to LDS in one pass: 2 chunks
                                                    // per thread, or 3 for longer rings (kNonFlushRowsLong).
                                                    constexpr int NT = StepTile<DV, DK, TL, SP, kNonFlushRows>::NT;
                                                    static_assert(NT == StepTile<DV, DK, TL, SP, kNonFlushRowsLong>::NT, "");
                                                    constexpr int rec_chunks = (DK + DV / SP) * (int)sizeof(R) / 16;
                                                    auto run = [&](auto rows_c) {
                                                        constexpr int ROWSP = decltype(rows_c)::value;
                                                        const auto fn = k_replay_step<FORM, DV, DK, TS, TR, TI, SP, TL, false,
                                                                                      ROWSP, true>;
                                                        const PersistShape ps =
                                                            persist_shape(reinterpret_cast<const void*>(fn), NT, lds,
                                                                          Deferred<DV / SP, DK, R>::BYTES,
                                                                          (int64_t)p->n_rows * p->n_heads * SP);
                                                        if (!ps.grid) return false;
                                                        StepParams q = *p;
                                                        q.meta_off = ps.meta_off;
                                                        q.defer_off = ps.defer_off;
                                                        q.defer_cap = ps.defer_cap;
                                                        hipLaunchKernelGGL(fn, dim3(ps.grid), dim3(NT), ps.lds, stream, q);
                                                        return true;
                                                    };
                                                    if (slots * rec_chunks <= record_chunks(kNonFlushRows) * NT) {
                                                        if (run(std::integral_constant<int, kNonFlushRows>{})) return;
                                                    } else if (slots * rec_chunks <= record_chunks(kNonFlushRowsLong) * NT) {
                                                        if (run(std::integral_constant<int, kNonFlushRowsLong>{})) return;
                                                    }
                                                }
                                            }
                                            // A step where every row flushes, with one fp32
                                            // checkpoint, runs its tiles in twice as many parts:
                                            // each workgroup folds half the rows, so the fold's
                                            // arithmetic hides behind more loads in flight.
                                            // Measured on MI355X at batch 256 (outputs and
                                            // checkpoints bit-identical): the Nemotron-3-Super
                                            // layer's flush step 429.9 -> 393.7 us, grouped keys
                                            // 393.5 -> 372.2, Gated DeltaNet 128 x 128 206.4 ->
                                            // 191.8; with an fp16 state (123.1 -> 126.7) or an
                                            // E4M3 read copy (458.8 -> 467.4) it is slower.
                                            if constexpr (!TWO && std::is_same<TS, tF32>::value &&
                                                          tile_ok<DV, DK, TL, 2 * SP>()) {
                                                if (hint == RS_FLUSH_ALL) {
                                                    constexpr int FSP = 2 * SP;
                                                    StepParams q = *p;
                                                    q.flush_hint = RS_FLUSH_UNKNOWN;
                                                    const dim3 fg = this->template grid<FSP>();
                                                    const dim3 fb(Tile<DV, DK, TL, FSP>::NT);
                                                    const size_t fl_lds = lds_need<DV / FSP, DK, R>(slots, L.L);
                                                    hipLaunchKernelGGL((k_replay_step<FORM, DV, DK, TS, TR, TI, FSP, TL>), fg, fb,
                                                                       fl_lds, stream, q);
                                                    return;
                                                }
                                            }
                                            if constexpr (!TWO) {
                                                // one launch over every row; the hint is not used
                                                // (a pair of launches on mixed steps and the kernel
                                                // without the fold measured slower here)
                                                StepParams q = *p;
                                                q.flush_hint = RS_FLUSH_UNKNOWN;
                                                hipLaunchKernelGGL((k_replay_step<FORM, DV, DK, TS, TR, TI, SP, TL>), grid<SP>(),
                                                                   block, lds, stream, q);
                                            } else {
                                                if (hint == RS_FLUSH_NONE || hint == RS_FLUSH_MIXED)
                                                    hipLaunchKernelGGL((k_replay_step<FORM, DV, DK, TS, TR, TI, SP, TL, false,
                                                                                      kNonFlushRows>),
                                                                       grid<SP>(),
                                                                       dim3(StepTile<DV, DK, TL, SP, kNonFlushRows>::NT),
                                                                       lds, stream, *p);
                                                if (hint != RS_FLUSH_NONE)
                                                    hipLaunchKernelGGL((k_replay_step<FORM, DV, DK, TS, TR, TI, SP, TL>),
                                                                       grid<SP>(), block, lds, stream, *p);
                                            }
                                        };
                                        if constexpr (SPW != SPB) {
                                            if (whole) go(std::integral_constant<int, SPW>{});
                                            else go(std::integral_constant<int, SPB>{});
                                        } else {
                                            go(std::integral_constant<int, SPB>{});
                                        }
                                    }
                                });
                            }
                        });
                    });
                });
            });
        });
        if (ok && p) err = hipGetLastError();
        return ok;
    }
};

}  // namespace

// Upper bound over the splits (a workgroup owning all d_v rows).
size_t lds_bytes(Kind kind, const rs_layer& layer) {
    if (kind == Kind::SpecVerify)
    {
        const int rb = layer.record_dtype == RS_F32 ? 4 : 2;
        if (layer.form == RS_GDN)
            return spec_gdn_lds_bytes(layer.L, layer.spec_T, layer.d_v, layer.d_k, rb,
                                      spec_mf(kGdn, layer.d_v, layer.d_k, layer.state_dtype == RS_F32, layer.spec_T));
        return spec_lds_bytes(layer.L, layer.spec_T, layer.d_v, layer.d_k, rb);
    }
    if (kind != Kind::ReplayStep && kind != Kind::Flush) return 0;
    const int slots = layer.spec_T > 0 ? layer.L : layer.L - 1;
    const size_t rb = layer.record_dtype == RS_F32 ? 4 : 2;
    return (size_t)slots * (layer.d_k + layer.d_v) * rb + sizeof(float) * (3 * (size_t)layer.L + 2 * layer.d_v + 4);
}

bool compiled(Kind kind, const rs_layer& layer) {
    Dispatch d{kind, layer, nullptr, nullptr};
    return d.run();
}

hipError_t launch(Kind kind, const rs_layer& layer, const StepParams& p, hipStream_t stream) {
    Dispatch d{kind, layer, &p, stream};
    if (!d.run()) return hipErrorInvalidValue;
    return d.err;
}

}  // namespace rs
