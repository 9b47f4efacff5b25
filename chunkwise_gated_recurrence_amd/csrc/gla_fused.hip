// gla_fused.hip -- the fused fp16 path for d_k = d_v = 64, chunk C = 64, on
// gfx950 (CDNA4) MFMA.
//
// One kernel evaluates the chunkwise form of key-only GLA (GTR summary page
// "GTR:门控Token循环实现高效稠密预测", section 前置知识 › Chunkwise(分块)并行; the
// operator of section 方法步骤详情 and of section 3.3 on the 0539edu.com page):
// per-chunk summaries U_c and decays d_c, the boundary scan
// S_[c+1] = Diag(d_c) S_[c] + U_c, and per-chunk outputs.
//
// Work decomposition. A sequence (one batch entry, one head) is cut into spans
// of SPAN consecutive chunks. A workgroup (4 waves) takes spans from a ticket
// counter, so a span's predecessors always hold smaller tickets and are being
// worked on by running workgroups (no deadlock whatever the residency). For its
// span it:
//   1. streams the span's chunks once from HBM (direction folded into the row
//      addresses: no transposed copies), stages fp16 tiles in LDS and computes,
//      from a zero state at the span start, every chunk's outputs (intra-chunk
//      scores on MFMA, kept on chip, times V; plus the running local state),
//      the span summary (D = product of gates, U = local final state), and
//      keeps outputs (registers) and q * 2^{b} tiles (LDS) on chip;
//   2. publishes (D, U), then looks back over its predecessors (decoupled
//      look-back: fold published summaries until a published inclusive state
//      is found) to obtain the true state S_in entering the span, and publishes
//      its own inclusive state;
//   3. adds the inter-span term (q_t * 2^{b_t}) Diag(2^{P_c}) S_in to the
//      on-chip outputs and stores them.
// While one workgroup looks back, other workgroups on the CU stream their
// chunks: the boundary scan overlaps output computation.
//
// Intra-chunk scores A[t,s] = sum_i q_ti k_si 2^{b_ti - b_si} (s <= t, b the
// inclusive prefix of log2 gates) are the product (Q 2^{B-r}) (K 2^{r-B})^T with
// a per-key-dim reference r at the middle of the chunk's range, valid when
// the range max_i (b_first,i - b_last,i) <= kGuard (log2 units): then every
// factor lies in [2^-8, 2^8] and fp16 keeps full precision. A chunk outside
// the guard (very strong decay) computes its scores exactly in fp32 on the
// vector ALU instead; every other step only ever multiplies by factors <= 1.
#include "gla_common.h"
#include "gla_launch.h"

namespace gtrgla {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;            // chunk length
constexpr int kD = 64;            // d_k = d_v
constexpr int kThreads = 256;     // 4 waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kGuard = 16.0f;   // max log2 range of a chunk for the factorised scores
constexpr int kTile = kC * kD;    // halves per LDS tile

constexpr uint32_t kAgg = 1, kIncl = 2;
// Look-back polls before a wave gives up on a predecessor (about a second).
constexpr unsigned int kMaxPolls = 1u << 24;

// ---------------------------------------------------------------------------
// LDS tiles: 64 rows x 64 halves, 128 B per row, in 16 B granules permuted by
// row so that 8 consecutive rows (operand reads) and rows 8 apart (transposing
// writes) both fall on distinct banks.
__device__ __forceinline__ int swz(int row, int col)
{
    const int g = (col >> 3) ^ ((row ^ (row >> 3)) & 7);
    return row * kD + (g << 3) + (col & 7);
}
__device__ __forceinline__ h8 ld8(const _Float16* t, int row, int col)
{
    return *reinterpret_cast<const h8*>(t + swz(row, col));
}
__device__ __forceinline__ void st8(_Float16* t, int row, int col, h8 x)
{
    *reinterpret_cast<h8*>(t + swz(row, col)) = x;
}
__device__ __forceinline__ void st4(_Float16* t, int row, int col, h4 x)
{
    *reinterpret_cast<h4*>(t + swz(row, col)) = x;
}

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

struct FusedArgs {
    const __half* q;
    const __half* k;
    const __half* v;
    const __half* lg;
    __half* out;
    float* final_state;
    unsigned long long* ctrl;   // [epoch:32 | tickets taken:32]
    unsigned long long* flags;  // [slot][4 waves]
    float* slots;               // [slot] { U 4096 | D 64 | S 4096 }
    int L, H, grid_h, grid_w, dir;
    int n_chunks;               // per sequence
    int n_spans;                // per sequence
    int n_seq;                  // B * H
    int total;                  // n_seq * n_spans
    float scale;
};

constexpr int kSlotFloats = kD * kD + kD + kD * kD;

// Row offset (in halves) of scan step t of sequence (b, h), or -1 past the end.
__device__ __forceinline__ long long row_offset(const FusedArgs& a, int b, int h, int t)
{
    if (t >= a.L) return -1;
    const int p = scan_to_spatial(t, a.L, a.grid_h, a.grid_w, a.dir);
    return (((long long)b * a.L + p) * a.H + h) * kD;
}

__device__ __forceinline__ u4 load_row(const __half* base, long long off, int ig)
{
    if (off < 0) return u4{0u, 0u, 0u, 0u};
    return __builtin_nontemporal_load(reinterpret_cast<const u4*>(base + off) + ig);
}

__device__ __forceinline__ void unpack8(u4 u, float* f)
{
    const __half2* h = reinterpret_cast<const __half2*>(&u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float2 x = __half22float2(h[e]);
        f[2 * e] = x.x;
        f[2 * e + 1] = x.y;
    }
}

__device__ __forceinline__ h8 pack8(const float* f)
{
    h8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (_Float16)f[e];
    return r;
}

struct ChunkRegs {
    u4 q[2], k[2], v[2], g[2];
};

__device__ __forceinline__ void load_chunk(const FusedArgs& a, int b, int h, int t0, int r0, int ig,
                                           ChunkRegs& R)
{
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const long long off = row_offset(a, b, h, t0 + r0 + 32 * hf);
        R.q[hf] = load_row(a.q, off, ig);
        R.k[hf] = load_row(a.k, off, ig);
        R.v[hf] = load_row(a.v, off, ig);
        R.g[hf] = load_row(a.lg, off, ig);
    }
}

// Shared memory of one workgroup.
template <int SPAN>
struct Smem {
    _Float16 Qt[SPAN][kTile];   // q * 2^{b} per chunk of the span (kept until the end)
    _Float16 QhSc[kTile];       // q * 2^{b - r}, then the chunk's scores [t][s]
    _Float16 KhOs[kTile];       // k * 2^{r - b}, then output staging [t][j]
    _Float16 KtT[kTile];        // (k * 2^{b_last - b})^T  [i][s]
    _Float16 VT[kTile];         // v^T                     [j][s]
    _Float16 ST[2][kTile];      // fp16 copy of a state, transposed [j][i]
    float tot[8][kD];           // per 8-row group sums of log2 gates
    float bfirst[kD], blast[kD];
    float P[SPAN + 1][kD];      // log2 decay from the span start to each chunk start
    int ticket;
    unsigned int epoch;
    int fail[4];
};

// ---------------------------------------------------------------------------
// Exact fp32 scores for one chunk (strong-decay fallback). Needs raw q and k
// rows staged in QhSc / KhOs and the fp32 prefix in Bf; writes wave w's score
// rows into QhSc over its own q rows, after all of them have been read.
__device__ void exact_scores(_Float16* QhSc, const _Float16* Kraw, const float* Bf, int w, int lane)
{
    const int t = 16 * w + (lane & 15);
    h4 res[4];
    for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = 16 * sb + 4 * (lane >> 4) + e;
            float acc = 0.f;
            if (sb <= w && s <= t) {
                for (int i = 0; i < kD; i += 8) {
                    const h8 qx = ld8(QhSc, t, i);
                    const h8 kx = ld8(Kraw, s, i);
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const float d = fminf(Bf[t * kD + i + u] - Bf[s * kD + i + u], 0.f);
                        acc += (float)qx[u] * (float)kx[u] * exp2f(d);
                    }
                }
            }
            res[sb][e] = (_Float16)acc;
        }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) st4(QhSc, t, 16 * sb + 4 * (lane >> 4), res[sb]);
}

template <int SPAN>
__global__ void __launch_bounds__(kThreads, (SPAN <= 2) ? 2 : 1) gla_fused_kernel(FusedArgs a)
{
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem<SPAN>& sm = *reinterpret_cast<Smem<SPAN>*>(smem_raw);

    const int tid = threadIdx.x;
    const int w = tid >> 6;          // wave
    const int lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;
    const int r0 = tid >> 3;         // row of this thread's first 16 B segment
    const int ig = tid & 7;          // 8-half column group

    for (;;) {
        // ---- take a ticket --------------------------------------------------
        __syncthreads();
        if (tid == 0) {
            const unsigned long long old = atomicAdd(a.ctrl, 1ull);
            const unsigned int cnt = (unsigned int)old;
            sm.ticket = (int)cnt;
            sm.epoch = (unsigned int)(old >> 32);
            const unsigned int last = (unsigned int)(a.total + gridDim.x) - 1u;
            if (cnt == last)  // every ticket of this launch is taken: reset, next epoch
                atomicAdd(a.ctrl, (1ull << 32) - (unsigned long long)(a.total + gridDim.x));
        }
        __syncthreads();
        const int ticket = sm.ticket;
        if (ticket >= a.total) break;
        const unsigned long long epoch = sm.epoch;

        const int j = ticket / a.n_seq;           // span index in its sequence
        const int seq = ticket - j * a.n_seq;
        const int b = seq / a.H, h = seq - (seq / a.H) * a.H;
        const int c_first = j * SPAN;
        const int n_c = min(SPAN, a.n_chunks - c_first);
        const long long slot = (long long)seq * a.n_spans + j;

        // ---- pass 1: local outputs and state over the span ----------------
        f4 O[SPAN][4];
        f4 S[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) S[n] = f4{0.f, 0.f, 0.f, 0.f};
        if (tid < kD) sm.P[0][tid] = 0.f;

        ChunkRegs cur, nxt;
        load_chunk(a, b, h, c_first * kC, r0, ig, cur);

#pragma unroll
        for (int c = 0; c < SPAN; ++c) {
#pragma unroll
            for (int n = 0; n < 4; ++n) O[c][n] = f4{0.f, 0.f, 0.f, 0.f};
            if (c >= n_c) continue;
            if (c + 1 < n_c) load_chunk(a, b, h, (c_first + c + 1) * kC, r0, ig, nxt);

            // -- log2 gates: inclusive prefix over the chunk's 64 rows.
            //    lanes 8 apart hold consecutive rows: three shuffle steps scan
            //    8 rows inside the wave, LDS combines the 8 row groups.
            float x[2][8];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                unpack8(cur.g[hf], x[hf]);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[hf][e] *= kLog2e;
            }
#pragma unroll
            for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float y = __shfl_up(x[hf][e], off, 64);
                        if (lane >= off) x[hf][e] += y;
                    }
            }
            if (lane >= 56) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int e = 0; e < 8; ++e) sm.tot[4 * hf + w][8 * ig + e] = x[hf][e];
            }
            if (tid < 8) {
#pragma unroll
                for (int e = 0; e < 8; ++e) sm.bfirst[8 * ig + e] = x[0][e];
            }
            __syncthreads();  // (A)

            float bl[8], ref[8];
            bool wide = false;
#pragma unroll
            for (int e = 0; e < 8; ++e) bl[e] = 0.f;
#pragma unroll
            for (int g = 0; g < 8; ++g) {
                const f4 t0 = *reinterpret_cast<const f4*>(&sm.tot[g][8 * ig]);
                const f4 t1 = *reinterpret_cast<const f4*>(&sm.tot[g][8 * ig + 4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bl[e] += t0[e];
                    bl[4 + e] += t1[e];
                    if (g < w) { x[0][e] += t0[e]; x[0][4 + e] += t1[e]; }
                    if (g < 4 + w) { x[1][e] += t0[e]; x[1][4 + e] += t1[e]; }
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float bf = sm.bfirst[8 * ig + e];
                ref[e] = 0.5f * (bf + bl[e]);
                wide |= (bf - bl[e]) > kGuard;
            }
            // x now holds the inclusive prefix b of the thread's two rows
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int row = r0 + 32 * hf;
                float qf[8], kf[8], vf[8], qh[8], kh[8], qt[8];
                unpack8(cur.q[hf], qf);
                unpack8(cur.k[hf], kf);
                unpack8(cur.v[hf], vf);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float Bv = x[hf][e];
                    qh[e] = qf[e] * exp2f(fminf(Bv - ref[e], 30.f));
                    kh[e] = kf[e] * exp2f(fminf(ref[e] - Bv, 30.f));
                    qt[e] = qf[e] * exp2f(Bv);
                    const float kt = kf[e] * exp2f(bl[e] - Bv);
                    sm.KtT[swz(8 * ig + e, row)] = (_Float16)kt;
                    sm.VT[swz(8 * ig + e, row)] = (_Float16)vf[e];
                }
                st8(sm.QhSc, row, 8 * ig, pack8(qh));
                st8(sm.KhOs, row, 8 * ig, pack8(kh));
                st8(sm.Qt[c], row, 8 * ig, pack8(qt));
            }
            if (tid < 8) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sm.blast[8 * ig + e] = bl[e];
                    sm.P[c + 1][8 * ig + e] = sm.P[c][8 * ig + e] + bl[e];
                }
            }
            const bool wave_wide = __any(wide);
            if (lane == 0) sm.fail[w] = wave_wide ? 1 : 0;
            __syncthreads();  // (B)

            const bool exact = sm.fail[0] | sm.fail[1] | sm.fail[2] | sm.fail[3];
            if (exact) {
                // Strong decay: stage raw q, k and the fp32 prefix, compute exact
                // scores, then restore the tiles the MFMA steps below need.
                float* Bf = reinterpret_cast<float*>(sm.KtT);   // KtT and VT: 16 KB
                __syncthreads();
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int row = r0 + 32 * hf;
                    st8(sm.QhSc, row, 8 * ig, __builtin_bit_cast(h8, cur.q[hf]));
                    st8(sm.KhOs, row, 8 * ig, __builtin_bit_cast(h8, cur.k[hf]));
#pragma unroll
                    for (int e = 0; e < 8; ++e) Bf[row * kD + 8 * ig + e] = x[hf][e];
                }
                __syncthreads();
                exact_scores(sm.QhSc, sm.KhOs, Bf, w, lane);
                __syncthreads();
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int row = r0 + 32 * hf;
                    float kf[8], vf[8];
                    unpack8(cur.k[hf], kf);
                    unpack8(cur.v[hf], vf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float kt = kf[e] * exp2f(bl[e] - x[hf][e]);
                        sm.KtT[swz(8 * ig + e, row)] = (_Float16)kt;
                        sm.VT[swz(8 * ig + e, row)] = (_Float16)vf[e];
                    }
                }
                __syncthreads();
            } else {
                // Scores, transposed: Sc^T[s][t] = sum_i Kh[s][i] Qh[t][i], for the
                // wave's 16 rows t and every s-tile up to the diagonal. Written as
                // Sc[t][s] over the wave's own Qh rows.
                const int t = 16 * w + lr;
                f4 sc[4];
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) {
                    sc[sb] = f4{0.f, 0.f, 0.f, 0.f};
                    if (sb <= w) {
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks)
                            sc[sb] = mfma(ld8(sm.KhOs, 16 * sb + lr, 32 * ks + 8 * lq),
                                          ld8(sm.QhSc, 16 * w + lr, 32 * ks + 8 * lq), sc[sb]);
                    }
                }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) {
                    h4 r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = 16 * sb + 4 * lq + e;
                        r[e] = (_Float16)((s <= t) ? sc[sb][e] : 0.f);
                    }
                    st4(sm.QhSc, t, 16 * sb + 4 * lq, r);
                }
            }
            __builtin_amdgcn_wave_barrier();

            // -- outputs of the wave's 16 rows: O^T[j][t] = sum_s VT[j][s] Sc[t][s]
            //    + sum_i ST[j][i] Qt[t][i] (local state entering the chunk).
            const int kmax = (w >= 2) ? 2 : 1;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (ks < kmax)
                        O[c][jt] = mfma(ld8(sm.VT, 16 * jt + lr, 32 * ks + 8 * lq),
                                        ld8(sm.QhSc, 16 * w + lr, 32 * ks + 8 * lq), O[c][jt]);
                if (c > 0) {
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        O[c][jt] = mfma(ld8(sm.ST[c & 1], 16 * jt + lr, 32 * ks + 8 * lq),
                                        ld8(sm.Qt[c], 16 * w + lr, 32 * ks + 8 * lq), O[c][jt]);
                }
            }

            // -- state: S[i][j] <- d_c[i] S[i][j] + sum_s KtT[i][s] VT[j][s],
            //    wave w owns rows i in [16w, 16w+16).
            float dc[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) dc[e] = exp2f(sm.blast[16 * w + 4 * lq + e]);
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
                for (int e = 0; e < 4; ++e) S[jt][e] *= dc[e];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    S[jt] = mfma(ld8(sm.KtT, 16 * w + lr, 32 * ks + 8 * lq),
                                 ld8(sm.VT, 16 * jt + lr, 32 * ks + 8 * lq), S[jt]);
            }
            if (c + 1 < n_c) {
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    h4 r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = (_Float16)S[jt][e];
                    st4(sm.ST[(c + 1) & 1], 16 * jt + lr, 16 * w + 4 * lq, r);
                }
                cur = nxt;
            }
        }
        __syncthreads();  // P[] complete

        // ---- pass 2: boundary scan (decoupled look-back), per wave -----------
        // Wave w handles state rows i in [16w, 16w+16); lane holds
        // S[16w + 4lq + e][16jt + lr].
        float* my_slot = a.slots + slot * kSlotFloats;
        unsigned long long* my_flags = a.flags + slot * 4;
        float Dspan[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) Dspan[e] = exp2f(sm.P[n_c][16 * w + 4 * lq + e]);
        f4 Sin[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) Sin[n] = f4{0.f, 0.f, 0.f, 0.f};
        const bool last_span = (j == a.n_spans - 1);

        if (j > 0) {
            // publish the span summary (U = local state, D), unless the
            // predecessor's inclusive state is already there
            unsigned long long f0 = __hip_atomic_load(a.flags + (slot - 1) * 4 + w,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const bool pred_ready = (f0 == ((epoch << 2) | kIncl));
            if (!pred_ready) {
                f4* U = reinterpret_cast<f4*>(my_slot) + (w * 4) * 64 + lane;
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) U[jt * 64] = S[jt];
                if (lr == 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) my_slot[kD * kD + 16 * w + 4 * lq + e] = Dspan[e];
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                if (lane == 0)
                    __hip_atomic_store(my_flags + w, (epoch << 2) | kAgg, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            // look back
            float accD[4] = {1.f, 1.f, 1.f, 1.f};
            f4 acc[4];
#pragma unroll
            for (int n = 0; n < 4; ++n) acc[n] = f4{0.f, 0.f, 0.f, 0.f};
            long long m = slot - 1;
            for (;;) {
                unsigned long long f;
                unsigned int polls = 0;
                for (;;) {
                    f = __hip_atomic_load(a.flags + m * 4 + w, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                    if ((f >> 2) == epoch && (f & 3)) break;
                    if (++polls > kMaxPolls) {
                        // never expected: record it and stop waiting (results are
                        // then wrong, but every wave still exits)
                        if (lane == 0) atomicOr(a.ctrl + 1, 1ull);
                        f = (epoch << 2) | kIncl;
                        m = -1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                if (m < 0) break;
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                const float* ms = a.slots + m * kSlotFloats;
                if ((f & 3) == kIncl) {
                    const f4* Sm = reinterpret_cast<const f4*>(ms + kD * kD + kD) + (w * 4) * 64 + lane;
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt) {
                        const f4 sv = Sm[jt * 64];
#pragma unroll
                        for (int e = 0; e < 4; ++e) Sin[jt][e] = accD[e] * sv[e] + acc[jt][e];
                    }
                    break;
                }
                const f4* Um = reinterpret_cast<const f4*>(ms) + (w * 4) * 64 + lane;
                float Dm[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) Dm[e] = ms[kD * kD + 16 * w + 4 * lq + e];
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    const f4 uv = Um[jt * 64];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[jt][e] += accD[e] * uv[e];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) accD[e] *= Dm[e];
                --m;
            }
        }
        // inclusive state after the span
        f4 Sout[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int e = 0; e < 4; ++e) Sout[jt][e] = Dspan[e] * Sin[jt][e] + S[jt][e];
        if (!last_span) {
            f4* Sp = reinterpret_cast<f4*>(my_slot + kD * kD + kD) + (w * 4) * 64 + lane;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) Sp[jt * 64] = Sout[jt];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            if (lane == 0)
                __hip_atomic_store(my_flags + w, (epoch << 2) | kIncl, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        } else if (a.final_state) {
            float* fs = a.final_state + (long long)seq * kD * kD;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    fs[(16 * w + 4 * lq + e) * kD + 16 * jt + lr] = Sout[jt][e];
        }

        // ---- pass 3: add the inter-span term, store ---------------------------
        const bool has_in = (j > 0);
#pragma unroll
        for (int c = 0; c < SPAN; ++c) {
            if (c >= n_c) continue;
            if (has_in) {
                // ST <- fp16(Diag(2^{P_c}) S_in), transposed [j][i]
                float pc[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) pc[e] = exp2f(sm.P[c][16 * w + 4 * lq + e]);
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    h4 r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = (_Float16)(pc[e] * Sin[jt][e]);
                    st4(sm.ST[0], 16 * jt + lr, 16 * w + 4 * lq, r);
                }
                __syncthreads();
#pragma unroll
                for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        O[c][jt] = mfma(ld8(sm.ST[0], 16 * jt + lr, 32 * ks + 8 * lq),
                                        ld8(sm.Qt[c], 16 * w + lr, 32 * ks + 8 * lq), O[c][jt]);
            }
            // stage O[t][j] (fp16, scaled) and store rows with 16 B per thread
            const int t = 16 * w + lr;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                h4 r;
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = (_Float16)(O[c][jt][e] * a.scale);
                st4(sm.KhOs, t, 16 * jt + 4 * lq, r);
            }
            __syncthreads();
            const int tc = (c_first + c) * kC;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int row = r0 + 32 * hf;
                const long long off = row_offset(a, b, h, tc + row);
                if (off >= 0) {
                    const h8 val = ld8(sm.KhOs, row, 8 * ig);
                    __builtin_nontemporal_store(__builtin_bit_cast(u4, val),
                                                reinterpret_cast<u4*>(a.out + off) + ig);
                }
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
bool fused_supported(const Shape& s)
{
    return s.d_k == kD && s.d_v == kD && s.chunk == kC;
}

static int device_cus()
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 256;
    return cus;
}

template <int SPAN>
static size_t smem_bytes()
{
    return sizeof(Smem<SPAN>);
}

template <int SPAN>
static int resident_per_cu()
{
    static int cached = 0;
    if (cached == 0) {
        const size_t sh = smem_bytes<SPAN>();
        int n = 0;
        if (hipFuncSetAttribute((const void*)gla_fused_kernel<SPAN>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gla_fused_kernel<SPAN>, kThreads, sh) !=
                hipSuccess || n < 1)
            n = 1;
        cached = n;
    }
    return cached;
}

static int resident_for_span(int span)
{
    switch (span) {
    case 1: return resident_per_cu<1>();
    case 2: return resident_per_cu<2>();
    case 4: return resident_per_cu<4>();
    default: return resident_per_cu<8>();
    }
}

FusedPlan fused_plan(const Shape& s, int span_override)
{
    FusedPlan p;
    const int total_chunks_seq = s.n_chunks;
    const long long n_seq = (long long)s.B * s.H;
    int span = span_override;
    if (span <= 0) {
        // One chunk per workgroup while the whole problem fits a few rounds of
        // resident workgroups; longer spans beyond, so that the look-back chain
        // of a sequence stays short.
        const long long chunks = n_seq * total_chunks_seq;
        span = (chunks <= 4LL * resident_for_span(1) * device_cus()) ? 1 : 4;
    }
    if (span != 1 && span != 2 && span != 4 && span != 8) span = 1;
    p.span = span;
    p.n_spans = (total_chunks_seq + span - 1) / span;
    const long long total = n_seq * p.n_spans;
    // persistent grid: no more workgroups than can be resident at once
    const long long resident = (long long)resident_for_span(span) * device_cus();
    p.grid = (int)(total < resident ? total : resident);
    return p;
}

size_t fused_workspace_bytes(const Shape& s, const FusedPlan& p)
{
    const size_t total = (size_t)s.B * s.H * p.n_spans;
    return 256 + total * 4 * sizeof(unsigned long long) + total * kSlotFloats * sizeof(float);
}

template <int SPAN>
static hipError_t launch_span(const FusedArgs& a, int grid, hipStream_t st)
{
    const size_t sh = smem_bytes<SPAN>();
    resident_per_cu<SPAN>();   // also raises the kernel's dynamic LDS limit
    hipLaunchKernelGGL(gla_fused_kernel<SPAN>, dim3(grid), dim3(kThreads), sh, st, a);
    return hipGetLastError();
}

hipError_t launch_fused(const void* q, const void* k, const void* v, const void* lg,
                        const Shape& s, const FusedPlan& p, void* out, float* final_state,
                        void* ws, hipStream_t st)
{
    FusedArgs a;
    a.q = (const __half*)q;
    a.k = (const __half*)k;
    a.v = (const __half*)v;
    a.lg = (const __half*)lg;
    a.out = (__half*)out;
    a.final_state = final_state;
    unsigned char* base = (unsigned char*)ws;
    const size_t total = (size_t)s.B * s.H * p.n_spans;
    a.ctrl = (unsigned long long*)base;
    a.flags = (unsigned long long*)(base + 256);
    a.slots = (float*)(base + 256 + total * 4 * sizeof(unsigned long long));
    a.L = s.L;
    a.H = s.H;
    a.grid_h = s.grid_h;
    a.grid_w = s.grid_w;
    a.dir = s.dir;
    a.n_chunks = s.n_chunks;
    a.n_spans = p.n_spans;
    a.n_seq = s.B * s.H;
    a.total = (int)total;
    a.scale = s.scale;
    switch (p.span) {
    case 1: return launch_span<1>(a, p.grid, st);
    case 2: return launch_span<2>(a, p.grid, st);
    case 4: return launch_span<4>(a, p.grid, st);
    default: return launch_span<8>(a, p.grid, st);
    }
}

}  // namespace gtrgla
