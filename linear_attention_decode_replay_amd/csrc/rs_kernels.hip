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

#include "rs_internal.h"

namespace rs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- dtypes --
struct tF32 { using S = float; };
struct tF16 { using S = _Float16; };
struct tBF16 { using S = uint16_t; };

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

// ------------------------------------------------------- lane-group sums --
// Sum N per-lane values over an aligned group of lanes (offsets OFF, OFF/2,
// ..., 1; gl = lane index within the group).  While more than one value is
// left, the lane whose OFF bit is set keeps the upper half of its values,
// its partner the lower half, and each adds the partner's copy of the half
// it keeps; with one value left, plain butterflies finish.  Afterwards the
// first xsum_left<N,G>() entries of v hold complete sums of original indices
// xsum_base<N,G>(gl) + i, identical across the lanes that differ only in
// xsum_dup_mask<N,G>() bits.
template <int N, int OFF>
__device__ __forceinline__ void xsum(float* v, int gl) {
    if constexpr (OFF > 0) {
        if constexpr (N > 1) {
            const bool up = (gl & OFF) != 0;
#pragma unroll
            for (int i = 0; i < N / 2; ++i) {
                const float send = up ? v[i] : v[i + N / 2];
                const float keep = up ? v[i + N / 2] : v[i];
                v[i] = keep + __shfl_xor(send, OFF);
            }
            xsum<N / 2, OFF / 2>(v, gl);
        } else {
            v[0] += __shfl_xor(v[0], OFF);
            xsum<1, OFF / 2>(v, gl);
        }
    }
}

template <int N, int G>
constexpr int xsum_left() {
    int n = N;
    for (int o = G / 2; o > 0 && n > 1; o >>= 1) n /= 2;
    return n;
}

template <int N, int G>
__device__ __forceinline__ int xsum_base(int gl) {
    int n = N, b = 0;
#pragma unroll
    for (int o = G / 2; o > 0 && n > 1; o >>= 1) {
        if (gl & o) b += n / 2;
        n /= 2;
    }
    return b;
}

template <int N, int G>
constexpr int xsum_dup_mask() {
    int n = N, m = 0;
    for (int o = G / 2; o > 0; o >>= 1) {
        if (n > 1) n /= 2;
        else m |= o;
    }
    return m;
}

// Plain butterfly sum of one value over the group; every lane gets the sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// ------------------------------------------------------------ tile shape --
template <int DV, int DK, class TS>
struct Tile {
    using S = typename TS::S;
    static constexpr int VEC = 16 / (int)sizeof(S);           // state elements per 16 B
    static constexpr int LPR = DK / VEC;                       // lanes per state row
    static constexpr int LOADS = DV * LPR;                     // 16-B chunks per tile
    static constexpr int NT = LOADS >= 2048 ? 256 : (LOADS >= 512 ? 128 : 64);
    static constexpr int RPP = NT / LPR;                       // rows per pass
    static constexpr int NR = DV / RPP;                        // passes per thread
    static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "lane group");
    static_assert(NT % LPR == 0 && DV % RPP == 0 && NR >= 1, "tile split");
    static_assert((NR & (NR - 1)) == 0, "passes must be a power of two");
};

constexpr int kMamba2 = RS_MAMBA2;
constexpr int kGdn = RS_GDN;

struct TileIds {
    int row, head;
    int64_t tile;
};

__device__ __forceinline__ TileIds tile_ids(const StepParams& p) {
    TileIds t;
    t.tile = blockIdx.x;
    t.row = (int)(t.tile / p.n_heads);
    t.head = (int)(t.tile - (int64_t)t.row * p.n_heads);
    return t;
}

__device__ __forceinline__ void count_error(const StepParams& p) {
    if (threadIdx.x == 0 && p.err) atomicAdd(p.err, 1);
}

// LDS carve-up shared by the step and flush kernels.
template <class R>
struct Lds {
    R* k;         // [slots][DK] buffered keys
    R* x;         // [slots][DV] buffered values
    float* lam;   // [L]  buffered log-decays
    float* e;     // [L]  per-record decay weight
    float* cq;    // [L]  k_j . q
    float* ck;    // [L]  k_j . k (Gated DeltaNet)
    float* y;     // [DV] C q
    float* yk;    // [DV] C k (Gated DeltaNet)
    float* v;     // [DV] current v
    float* u;     // [DV] current corrected value d (Gated DeltaNet)
    float* sc;    // [4]  G, k . q
};

template <int DV, int DK, class R>
__device__ __forceinline__ Lds<R> carve(char* smem, int slots, int L) {
    Lds<R> s;
    s.k = reinterpret_cast<R*>(smem);
    s.x = s.k + (int64_t)slots * DK;
    float* f = reinterpret_cast<float*>(s.x + (int64_t)slots * DV);
    s.lam = f;
    s.e = s.lam + L;
    s.cq = s.e + L;
    s.ck = s.cq + L;
    s.y = s.ck + L;
    s.yk = s.y + DV;
    s.v = s.yk + DV;
    s.u = s.v + DV;
    s.sc = s.u + DV;
    return s;
}

template <int DV, int DK, class R>
constexpr size_t lds_need(int slots, int L) {
    return (size_t)slots * (DK + DV) * sizeof(R) + sizeof(float) * (4 * (size_t)L + 4 * DV + 4);
}

// Copy records 0..w-1 (keys then values) into LDS in 16-byte chunks.  The
// first RC chunks per thread are loaded by rec_issue() before the caller
// issues its checkpoint loads and written by rec_commit() afterwards; any
// remainder (only when w * record bytes exceeds RC * NT * 16) is copied by
// rec_commit() directly.
template <int DV, int DK, class R, int NT, int RC>
struct RecordCopy {
    static constexpr int KCH = DK * (int)sizeof(R) / 16;
    static constexpr int XCH = DV * (int)sizeof(R) / 16;
    static_assert(DK * sizeof(R) % 16 == 0 && DV * sizeof(R) % 16 == 0, "record rows");
    u32x4 buf[RC];
    int nk, n;

    __device__ __forceinline__ void issue(const R* rk, const R* rx, int w) {
        nk = w * KCH;
        n = nk + w * XCH;
#pragma unroll
        for (int u = 0; u < RC; ++u) {
            const int i = u * NT + (int)threadIdx.x;
            if (i < n)
                buf[u] = i < nk ? reinterpret_cast<const u32x4*>(rk)[i]
                                : reinterpret_cast<const u32x4*>(rx)[i - nk];
        }
    }
    __device__ __forceinline__ void commit(const R* rk, const R* rx, R* sk, R* sx) {
#pragma unroll
        for (int u = 0; u < RC; ++u) {
            const int i = u * NT + (int)threadIdx.x;
            if (i < n) {
                if (i < nk) reinterpret_cast<u32x4*>(sk)[i] = buf[u];
                else reinterpret_cast<u32x4*>(sx)[i - nk] = buf[u];
            }
        }
        for (int i = RC * NT + (int)threadIdx.x; i < n; i += NT) {
            if (i < nk) reinterpret_cast<u32x4*>(sk)[i] = reinterpret_cast<const u32x4*>(rk)[i];
            else reinterpret_cast<u32x4*>(sx)[i - nk] = reinterpret_cast<const u32x4*>(rx)[i - nk];
        }
    }
};

// Decay weights: thread j < w writes e_j = exp(base + sum_{j<l<w} lam_l);
// thread w writes G = exp(base + sum_{l<w} lam_l) to sc[0].
__device__ __forceinline__ void decay_weights(float* lam, float* e, float* sc, int w, float base) {
    const int j = threadIdx.x;
    if (j <= w) {
        float acc = base;
        for (int l = (j == w ? 0 : j + 1); l < w; ++l) acc += lam[l];
        if (j < w) e[j] = expf(acc);
        else sc[0] = expf(acc);
    }
}

// ----------------------------------------------------- replay decode step --
template <int FORM, int DV, int DK, class TS, class TR, class TI>
__global__ __launch_bounds__((Tile<DV, DK, TS>::NT)) void k_replay_step(const StepParams p) {
    using T = Tile<DV, DK, TS>;
    using S = typename TS::S;
    using R = typename TR::S;
    using I = typename TI::S;
    constexpr int NT = T::NT, VEC = T::VEC, LPR = T::LPR, RPP = T::RPP, NR = T::NR;
    constexpr int NV = FORM == kGdn ? 2 * NR : NR;  // row sums per thread

    const TileIds id = tile_ids(p);
    const int blk = p.block_table[id.row];
    if (blk < 0) return;  // padding row
    const int w = p.write_pos[id.row];
    if (blk >= p.n_blocks || w < 0 || w > p.slots) {
        count_error(p);
        return;
    }
    const bool fl = (w == p.slots) || (p.flush && p.flush[id.row]);

    const int tid = threadIdx.x;
    const int cc = tid % LPR;  // column chunk
    const int rg = tid / LPR;  // row within a pass

    char* base = p.pool + (int64_t)blk * p.block_bytes;
    S* ck = reinterpret_cast<S*>(base + p.ckpt_off) + (int64_t)id.head * (DV * DK);
    R* rx = reinterpret_cast<R*>(base + p.recx_off) + (int64_t)id.head * p.slots * DV;
    R* rk = reinterpret_cast<R*>(base + p.reck_off) + (int64_t)id.head * p.slots * DK;
    float* rl = reinterpret_cast<float*>(base + p.reclam_off) + (int64_t)id.head * p.slots;
    const I* qp = static_cast<const I*>(p.q) + id.row * p.qs_r + id.head * p.qs_h;
    const I* kp = static_cast<const I*>(p.k) + id.row * p.ks_r + id.head * p.ks_h;
    const I* vp = static_cast<const I*>(p.v) + id.row * p.vs_r + id.head * p.vs_h;
    const float lam = p.lam[id.tile];

    extern __shared__ __attribute__((aligned(16))) char smem[];
    const Lds<R> s = carve<DV, DK, R>(smem, p.slots, p.L);

    // Records first (small), then the checkpoint stream, then the token.
    RecordCopy<DV, DK, R, NT, 2> rec;
    rec.issue(rk, rx, w);
    u32x4 cb[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r)
        cb[r] = *reinterpret_cast<const u32x4*>(ck + (int64_t)(r * RPP + rg) * DK + cc * VEC);
    float qv[VEC], kv[VEC];
    load_f<TI, VEC>(qp + cc * VEC, qv);
    load_f<TI, VEC>(kp + cc * VEC, kv);
    for (int i = tid; i < DV; i += NT) s.v[i] = to_f<TI>(vp[i]);
    if (tid < w) s.lam[tid] = rl[tid];

    // Non-flush append of what does not depend on the state: lam and k for
    // both forms, and v for Mamba-2 (Gated DeltaNet appends d further down).
    if (!fl) {
        for (int i = tid; i < DK; i += NT) rk[(int64_t)w * DK + i] = from_f<TR>(to_f<TI>(kp[i]));
        if constexpr (FORM == kMamba2)
            for (int i = tid; i < DV; i += NT) rx[(int64_t)w * DV + i] = from_f<TR>(to_f<TI>(vp[i]));
        if (tid == 0) rl[w] = lam;
    }

    rec.commit(rk, rx, s.k, s.x);
    __syncthreads();

    decay_weights(s.lam, s.e, s.sc, w, FORM == kMamba2 ? lam : 0.0f);

    // Record dot products: lane group rg takes records rg, rg + RPP, ...;
    // index w stands for the current token (k . q).
    const int rounds = (w + RPP) / RPP;
    for (int it = 0; it < rounds; ++it) {
        const int j = it * RPP + rg;
        float kj[VEC];
        if (j < w) {
            load_f<TR, VEC>(s.k + (int64_t)j * DK + cc * VEC, kj);
        } else {
#pragma unroll
            for (int c = 0; c < VEC; ++c) kj[c] = kv[c];
        }
        float pq = 0.f, pk = 0.f;
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            pq += kj[c] * qv[c];
            if constexpr (FORM == kGdn) pk += kj[c] * kv[c];
        }
        pq = group_sum<LPR>(pq);
        if constexpr (FORM == kGdn) pk = group_sum<LPR>(pk);
        if (cc == 0 && j <= w) {
            if (j < w) {
                s.cq[j] = pq;
                if constexpr (FORM == kGdn) s.ck[j] = pk;
            } else {
                s.sc[1] = pq;
            }
        }
    }

    // Checkpoint GEMV: C q (and C k for Gated DeltaNet) from one register copy.
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
        acc[r] = a;
        if constexpr (FORM == kGdn) acc[NR + r] = b;
    }
    xsum<NV, LPR / 2>(acc, cc);
    {
        constexpr int left = xsum_left<NV, LPR>();
        const int b0 = xsum_base<NV, LPR>(cc);
        if ((cc & xsum_dup_mask<NV, LPR>()) == 0) {
#pragma unroll
            for (int i = 0; i < left; ++i) {
                const int idx = b0 + i;
                const int r = idx % NR;
                float* dst = (FORM == kGdn && idx >= NR) ? s.yk : s.y;
                dst[r * RPP + rg] = acc[i];
            }
        }
    }
    __syncthreads();

    const float G = s.sc[0];
    const float kq = s.sc[1];
    const float alpha = expf(lam);  // used by Gated DeltaNet only
    for (int i = tid; i < DV; i += NT) {
        float* o = p.out + id.tile * DV;
        if constexpr (FORM == kMamba2) {
            float acc_o = G * s.y[i];
            for (int j = 0; j < w; ++j) acc_o += (s.e[j] * s.cq[j]) * to_f<TR>(s.x[(int64_t)j * DV + i]);
            acc_o += kq * s.v[i];
            o[i] = acc_o;
        } else {
            float aq = G * s.y[i], ak = G * s.yk[i];
            for (int j = 0; j < w; ++j) {
                const float xj = to_f<TR>(s.x[(int64_t)j * DV + i]);
                aq += (s.e[j] * s.cq[j]) * xj;
                ak += (s.e[j] * s.ck[j]) * xj;
            }
            const float d = p.beta[id.tile] * (s.v[i] - alpha * ak);
            o[i] = alpha * aq + kq * d;
            if (fl) s.u[i] = d;
            else rx[(int64_t)w * DV + i] = from_f<TR>(d);
        }
    }

    if (!fl) return;  // uniform across the workgroup

    // Flush: fold records and the current token into the registers holding
    // the tile, store once.
    //   Mamba-2:  C' = G C + sum_j e_j x_j k_j^T + v k^T
    //   GDN:      C' = alpha P C + sum_j alpha p_j d_j k_j^T + d k^T
    if constexpr (FORM == kGdn) __syncthreads();  // d in LDS
    const float gc = FORM == kMamba2 ? G : alpha * G;
    const float ge = FORM == kMamba2 ? 1.0f : alpha;
    const float* u = FORM == kMamba2 ? s.v : s.u;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const float ur = u[r * RPP + rg];
#pragma unroll
        for (int c = 0; c < VEC; ++c) cf[r][c] = gc * cf[r][c] + ur * kv[c];
    }
    for (int j = 0; j < w; ++j) {
        float kj[VEC];
        load_f<TR, VEC>(s.k + (int64_t)j * DK + cc * VEC, kj);
        const float ej = ge * s.e[j];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const float f = ej * to_f<TR>(s.x[(int64_t)j * DV + r * RPP + rg]);
#pragma unroll
            for (int c = 0; c < VEC; ++c) cf[r][c] += f * kj[c];
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
        *reinterpret_cast<u32x4*>(ck + (int64_t)(r * RPP + rg) * DK + cc * VEC) = pack16<TS>(cf[r]);
}

// ------------------------------------------------ conventional decode step --
template <int FORM, int DV, int DK, class TS, class TI>
__global__ __launch_bounds__((Tile<DV, DK, TS>::NT)) void k_conventional_step(const StepParams p) {
    using T = Tile<DV, DK, TS>;
    using S = typename TS::S;
    using I = typename TI::S;
    constexpr int NT = T::NT, VEC = T::VEC, LPR = T::LPR, RPP = T::RPP, NR = T::NR;
    constexpr int NV = FORM == kGdn ? 2 * NR : NR;

    const TileIds id = tile_ids(p);
    const int blk = p.block_table[id.row];
    if (blk < 0) return;
    if (blk >= p.n_blocks) {
        count_error(p);
        return;
    }
    const int tid = threadIdx.x;
    const int cc = tid % LPR;
    const int rg = tid / LPR;

    char* base = p.pool + (int64_t)blk * p.block_bytes;
    S* ck = reinterpret_cast<S*>(base + p.ckpt_off) + (int64_t)id.head * (DV * DK);
    const I* qp = static_cast<const I*>(p.q) + id.row * p.qs_r + id.head * p.qs_h;
    const I* kp = static_cast<const I*>(p.k) + id.row * p.ks_r + id.head * p.ks_h;
    const I* vp = static_cast<const I*>(p.v) + id.row * p.vs_r + id.head * p.vs_h;

    __shared__ float s_y[DV], s_yk[DV], s_u[DV];

    u32x4 cb[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r)
        cb[r] = *reinterpret_cast<const u32x4*>(ck + (int64_t)(r * RPP + rg) * DK + cc * VEC);
    float qv[VEC], kv[VEC];
    load_f<TI, VEC>(qp + cc * VEC, qv);
    load_f<TI, VEC>(kp + cc * VEC, kv);
    const float alpha = expf(p.lam[id.tile]);

    float kq = 0.f;
#pragma unroll
    for (int c = 0; c < VEC; ++c) kq += kv[c] * qv[c];
    kq = group_sum<LPR>(kq);

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
        acc[r] = a;
        if constexpr (FORM == kGdn) acc[NR + r] = b;
    }
    xsum<NV, LPR / 2>(acc, cc);
    {
        constexpr int left = xsum_left<NV, LPR>();
        const int b0 = xsum_base<NV, LPR>(cc);
        if ((cc & xsum_dup_mask<NV, LPR>()) == 0) {
#pragma unroll
            for (int i = 0; i < left; ++i) {
                const int idx = b0 + i;
                float* dst = (FORM == kGdn && idx >= NR) ? s_yk : s_y;
                dst[(idx % NR) * RPP + rg] = acc[i];
            }
        }
    }
    __syncthreads();

    // o = S_t q = alpha (S_{t-1} q) + (k . q) u, with u = v (Mamba-2) or the
    // corrected value d = beta (v - alpha S_{t-1} k) (Gated DeltaNet).
    for (int i = tid; i < DV; i += NT) {
        const float vi = to_f<TI>(vp[i]);
        float ui = vi;
        if constexpr (FORM == kGdn) ui = p.beta[id.tile] * (vi - alpha * s_yk[i]);
        p.out[id.tile * DV + i] = alpha * s_y[i] + kq * ui;
        s_u[i] = ui;
    }
    __syncthreads();

    // S_t = alpha S_{t-1} + u k^T, stored every step.
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const float ur = s_u[r * RPP + rg];
#pragma unroll
        for (int c = 0; c < VEC; ++c) cf[r][c] = alpha * cf[r][c] + ur * kv[c];
        *reinterpret_cast<u32x4*>(ck + (int64_t)(r * RPP + rg) * DK + cc * VEC) = pack16<TS>(cf[r]);
    }
}

// ------------------------------------------------------ token-less flush --
template <int DV, int DK, class TS, class TR>
__global__ __launch_bounds__((Tile<DV, DK, TS>::NT)) void k_replay_flush(const StepParams p) {
    using T = Tile<DV, DK, TS>;
    using S = typename TS::S;
    using R = typename TR::S;
    constexpr int NT = T::NT, VEC = T::VEC, LPR = T::LPR, RPP = T::RPP, NR = T::NR;

    const TileIds id = tile_ids(p);
    const int blk = p.block_table[id.row];
    if (blk < 0 || !p.flush[id.row]) return;
    const int w = p.write_pos[id.row];
    if (blk >= p.n_blocks || w < 0 || w > p.slots) {
        count_error(p);
        return;
    }
    if (w == 0) return;  // nothing buffered: the checkpoint is the state

    const int tid = threadIdx.x;
    const int cc = tid % LPR;
    const int rg = tid / LPR;
    char* base = p.pool + (int64_t)blk * p.block_bytes;
    S* ck = reinterpret_cast<S*>(base + p.ckpt_off) + (int64_t)id.head * (DV * DK);
    const R* rx = reinterpret_cast<const R*>(base + p.recx_off) + (int64_t)id.head * p.slots * DV;
    const R* rk = reinterpret_cast<const R*>(base + p.reck_off) + (int64_t)id.head * p.slots * DK;
    const float* rl = reinterpret_cast<const float*>(base + p.reclam_off) + (int64_t)id.head * p.slots;

    extern __shared__ __attribute__((aligned(16))) char smem[];
    const Lds<R> s = carve<DV, DK, R>(smem, p.slots, p.L);

    RecordCopy<DV, DK, R, NT, 2> rec;
    rec.issue(rk, rx, w);
    u32x4 cb[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r)
        cb[r] = *reinterpret_cast<const u32x4*>(ck + (int64_t)(r * RPP + rg) * DK + cc * VEC);
    if (tid < w) s.lam[tid] = rl[tid];
    rec.commit(rk, rx, s.k, s.x);
    __syncthreads();
    decay_weights(s.lam, s.e, s.sc, w, 0.0f);
    __syncthreads();

    // C' = G C + sum_j e_j x_j k_j^T  with G = exp(sum_{l<w} lam_l).
    const float G = s.sc[0];
    float cf[NR][VEC];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        unpack16<TS>(cb[r], cf[r]);
#pragma unroll
        for (int c = 0; c < VEC; ++c) cf[r][c] *= G;
    }
    for (int j = 0; j < w; ++j) {
        float kj[VEC];
        load_f<TR, VEC>(s.k + (int64_t)j * DK + cc * VEC, kj);
        const float ej = s.e[j];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const float f = ej * to_f<TR>(s.x[(int64_t)j * DV + r * RPP + rg]);
#pragma unroll
            for (int c = 0; c < VEC; ++c) cf[r][c] += f * kj[c];
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
        *reinterpret_cast<u32x4*>(ck + (int64_t)(r * RPP + rg) * DK + cc * VEC) = pack16<TS>(cf[r]);
}

// ------------------------------------------------------------ state reset --
template <int DV, int DK, class TS>
__global__ __launch_bounds__((Tile<DV, DK, TS>::NT)) void k_state_reset(const StepParams p) {
    using T = Tile<DV, DK, TS>;
    using S = typename TS::S;
    constexpr int NT = T::NT, NR = T::NR;
    const TileIds id = tile_ids(p);
    const int blk = p.block_table[id.row];
    if (blk < 0 || !p.mask[id.row]) return;
    if (blk >= p.n_blocks) {
        count_error(p);
        return;
    }
    S* ck = reinterpret_cast<S*>(p.pool + (int64_t)blk * p.block_bytes + p.ckpt_off) +
            (int64_t)id.head * (DV * DK);
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int r = 0; r < NR; ++r) reinterpret_cast<u32x4*>(ck)[r * NT + threadIdx.x] = z;
}

// -------------------------------------------------------------- dispatch --
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
bool with_form(int form, F&& f) {
    if (form == RS_MAMBA2) { f(std::integral_constant<int, kMamba2>{}); return true; }
    if (form == RS_GDN) { f(std::integral_constant<int, kGdn>{}); return true; }
    return false;
}

struct Dispatch {
    Kind kind;
    const rs_layer& L;
    const StepParams* p;   // nullptr: only check that a kernel exists
    hipStream_t stream;
    hipError_t err = hipSuccess;

    bool run() {
        const int slots = L.L - 1;
        bool ok = false;
        with_shape(L.d_v, L.d_k, [&](auto dv_c, auto dk_c) {
            constexpr int DV = decltype(dv_c)::value, DK = decltype(dk_c)::value;
            with_state(L.state_dtype, [&](auto ts) {
                using TS = decltype(ts);
                using T = Tile<DV, DK, TS>;
                const dim3 block(T::NT);
                const dim3 grid(p ? (unsigned)((int64_t)p->n_rows * p->n_heads) : 1u);
                if (kind == Kind::Reset) {
                    ok = true;
                    if (p) hipLaunchKernelGGL((k_state_reset<DV, DK, TS>), grid, block, 0, stream, *p);
                    return;
                }
                if (kind == Kind::ConventionalStep) {
                    with_form(L.form, [&](auto f_c) {
                        constexpr int FORM = decltype(f_c)::value;
                        with_io(L.io_dtype, [&](auto ti) {
                            using TI = decltype(ti);
                            ok = true;
                            if (p) hipLaunchKernelGGL((k_conventional_step<FORM, DV, DK, TS, TI>), grid, block, 0, stream, *p);
                        });
                    });
                    return;
                }
                with_record(L.record_dtype, [&](auto tr) {
                    using TR = decltype(tr);
                    using R = typename TR::S;
                    const size_t lds = lds_need<DV, DK, R>(slots, L.L);
                    if (kind == Kind::Flush) {
                        ok = true;
                        if (p) hipLaunchKernelGGL((k_replay_flush<DV, DK, TS, TR>), grid, block, lds, stream, *p);
                        return;
                    }
                    with_form(L.form, [&](auto f_c) {
                        constexpr int FORM = decltype(f_c)::value;
                        with_io(L.io_dtype, [&](auto ti) {
                            using TI = decltype(ti);
                            ok = true;
                            if (p) hipLaunchKernelGGL((k_replay_step<FORM, DV, DK, TS, TR, TI>), grid, block, lds, stream, *p);
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

size_t lds_bytes(Kind kind, const rs_layer& layer) {
    if (kind != Kind::ReplayStep && kind != Kind::Flush) return 0;
    const int slots = layer.L - 1;
    const size_t rb = layer.record_dtype == RS_F32 ? 4 : 2;
    return (size_t)slots * (layer.d_k + layer.d_v) * rb + sizeof(float) * (4 * (size_t)layer.L + 4 * layer.d_v + 4);
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
