// kda_fused_pipe.hip -- the pipelined fused chunked KDA forward for gfx950
// (bf16 q/k/v).
//
// Same chunk algebra as the serial kernel (kda_fused_serial.hip), organised as
// a two-stage pipeline inside each workgroup:
//   * NS "state" waves each own 16 V columns of the 128 x 128 fp32 state of one
//     (sequence, head) and run the sequential part of chunk i:
//        P = (K*gamma) S,  Delta = (I + A)^{-1} Diag(beta) (V - P),
//        O = (Q*gamma) S + M Delta,  S <- Diag(gamma_last) S + Kt^T Delta;
//     before the mid-chunk barrier they also invert the two diagonal blocks
//     of I + A of chunk i (fp32 MFMA), from A that the helpers left in LDS.
//   * NH "helper" waves prepare chunk i+1 at the same time. A helper lane owns
//     two channels of four consecutive tokens; one wave holds all eight
//     segments of its channels, so the in-chunk log-gate scan needs no
//     workgroup synchronisation. Before the mid-chunk barrier the lanes form
//     every gated factor of their eight elements (VALU work); after it the
//     helpers build the gated K K^T blocks (A) and the gated Q K^T blocks (M)
//     on bf16 MFMA and form the state waves' fp16 operands, writing them into
//     the other half of a double-buffered LDS area.
// So the element work of chunk i+1 overlaps the inversion and the products
// with the old state of chunk i, and the block products of chunk i+1 overlap
// the solve and state update of chunk i. Two workgroup barriers per chunk: the
// mid-chunk one, and one at the end, which hands the operand buffers over.
// Two helper waves share each SIMD with one state wave: a single wave issues a
// VALU instruction at most every other slot, so the helpers' element work
// needs two waves per SIMD.
// The split into a chunk-parallel preparation and a sequential recurrence is
// the pages' two-kernel design (toolarium.ru page, section "Где ограничения
// прямо сейчас"); here the two run concurrently on one CU so that each input
// byte crosses HBM once. The same halves as two kernels (kda_prep_pipe,
// kda_recur_pipe, at the end of this file) are kept as a measured ablation.
//
// Precision: the gated factors of A and M are two-term bf16 splits on both
// sides (three MFMA terms per product, about 16 significant bits, fp32
// range). The products with the state reuse those key and query factors:
// (K*gamma) S = Ka (Diag(e^Gamma_ref) S), and likewise for Q, with the scaled
// state split into two bf16 terms as well, so the inter-chunk terms carry the
// same 16 bits whatever the state's magnitude. Kt is single fp16, beta (V - P)
// and Delta two-term fp16.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace pipe {

constexpr int C = 32;          // chunk length (two 16-token sub-blocks)
constexpr int NH = 8;          // helper waves, 16 channels each
// NS state waves (16 V columns each) per workgroup: 8, 4, 2 or 1, so a
// (sequence, head) is split over P = 1, 2, 4 or 8 workgroups. Every split
// computes the same values in the same order per column; a finer split only
// repeats the helper work, which pays when there are too few chains to fill
// the chip. With more chains than the chip holds at P = 2, P = 1 (sixteen
// waves, four per SIMD) does each chain's helper work once.
template <int NS>
struct Split {
    static constexpr int NT = 64 * (NS + NH);   // threads per workgroup
    static constexpr int VB = 16 * NS;          // V columns per workgroup
    static constexpr int P = D / VB;            // workgroups per (sequence, head)
};
constexpr int SEG = 4;         // tokens per helper lane
constexpr int NSEG = C / SEG;  // segments per chunk (lanes 8*seg + cp)
constexpr int TP = C;          // row length of a 2-byte [row][32] array (unpadded, see tcol)
constexpr float LOG2E = 1.4426950408889634f;
constexpr int MAX_RANKED = 64;  // varlen batches up to this many sequences run longest first
static_assert(NH * 16 == D && NSEG * 8 == 64, "helper lanes: 8 channel pairs x 8 segments per wave");

// LDS layouts. A 16-byte LDS read (ds_read_b128) serves a wave in four
// cycles of sixteen lanes: lanes 0-31, then 32-63, each half split by the
// parity of lane bits 2-4; the sixteen pieces of one cycle must fall on
// different 16-byte bank groups of a 256-byte line (64 banks of 4 bytes).
// 4-byte accesses serve 32 lanes a cycle over 32 banks (a 128-byte line).
// (Both rules measured on the chip with one access pattern per dispatch and
// the LDS bank-conflict counter.) An MFMA operand read, lane (row l16,
// 16-byte piece grp), therefore puts rows 0-3 and 12-15 of one piece in the
// same cycle as rows 4-11 of the next piece. Rows are unpadded and each
// row permutes its 16-byte pieces by an XOR, chosen so that those reads and
// the writers' stores use every bank once per cycle.
//
// [token][channel] arrays (128 positions per row): piece q of row r sits at
// piece q ^ fswz(r), fswz(r) = r0 | r2 << 1 | r3 << 2 | r1 << 3 (bits of r).
// A helper store instruction (eight channel pairs that fill all four words of
// two pieces, rows 4s + t for four s) then meets 32 distinct banks, and an
// operand read of 16 rows meets 16 distinct bank groups in each cycle.
__device__ __forceinline__ constexpr int fswz(int r) {
    return (r & 1) | ((r >> 1) & 2) | ((r >> 1) & 4) | ((r << 2) & 8);
}
// Element index of (row r, position p) in a [token][channel] array.
__device__ __forceinline__ constexpr int fidx(int r, int p) {
    return r * D + ((((p >> 3) ^ fswz(r)) << 3) | (p & 7));
}
constexpr int ROWS32 = C * D;
// Column of (row r, position p) in a [row][32] 2-byte array: the second and
// third pieces trade places in rows 8-15 of each 16, which makes the 16-row
// operand reads conflict-free.
__device__ __forceinline__ constexpr int tcol(int r, int p) {
    return (((p >> 3) ^ ((r >> 2) & 2)) << 3) | (p & 7);
}
// Column of (row r, position p) in K~^T ([channel][32 tokens]): pieces are
// permuted by 2 * r2 | r4. Its writers store one 16-byte piece per lane, and
// 16-byte stores serve eight consecutive lanes a cycle over 32 banks (a
// 128-byte line; measured like the reads): the eight rows of such a cycle
// alternate in parity and their four same-parity rows differ in bits 2 and 4.
// The 16-row operand reads stay conflict-free as well.
__device__ __forceinline__ constexpr int kcol(int r, int p) {
    return (((p >> 3) ^ (((r >> 1) & 2) | ((r >> 4) & 1))) << 3) | (p & 7);
}
// First channel of a helper lane's channel pair: wave hw covers channels
// 8h .. 8h+7 and 16+8h .. 16+8h+7 of its 32-group (h = hw & 1), whose kperm
// positions fill two whole 16-byte pieces of a row (see fidx).
__device__ __forceinline__ constexpr int hchan(int hw, int cp) {
    return 32 * (hw >> 1) + 8 * (hw & 1) + 2 * (cp & 3) + 16 * (cp >> 2);
}

// 2^x as one v_exp_f32. Every argument here lies within [-120, 60] (log2
// units of at most 24 decay steps with g >= -5) or underflows harmlessly:
// such a factor only multiplies a product that is itself below 2^-120.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer access to one chunk of a [row][H][128] tensor: the resource
// starts at the chunk's first row (this head) and ends after its last valid
// row, so reads of rows past the end return zero and writes there are dropped.
// Word 3 is the gfx9 raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* p, long long elem_off, int elem_bytes,
                                                             int nv, uint32_t row_elems, int valid_elems) {
    const char* base = static_cast<const char*>(p) + elem_off * elem_bytes;
    const int nbytes = nv > 0 ? ((nv - 1) * (int)row_elems + valid_elems) * elem_bytes : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, nbytes, 0x00020000);
}

__device__ __forceinline__ uint32_t pack_bf16(float x0, float x1) {
    bf16x2 h = {(__bf16)x0, (__bf16)x1};
    return __builtin_bit_cast(uint32_t, h);
}

// Value of the neighbouring lane (l ^ 1).
__device__ __forceinline__ float swap_pair(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}

// Operands of one chunk for the state waves (double-buffered).
struct alignas(16) Ops {
    _Float16 KtT[D][TP];            // (K * exp(Gamma_last - Gamma))^T, [channel][kperm(token)]
    _Float16 Tm[C][TP];             // block-diagonal (I + A)^{-1}, [row][kperm(col)]
    _Float16 A10[16][TP];           // A rows 16-31, cols 0-15, [row][kperm(col)]
    _Float16 M[2][C][TP];           // lower gated Q K^T, [hi, lo][row][kperm(col)]
    float Af[2][16][16];            // diagonal blocks A00, A11 in fp32, [row][col]
    float gl[D];                    // exp(Gamma_last), the chunk's decay per channel
    float c1[D];                    // exp(Gamma_ref), per channel
    float beta[C];
};

// Gated factors of one chunk, referenced to Gamma at the chunk's token 15
// (Gamma_ref): the key and query factors of A and M, and (with the state
// scaled by exp(Gamma_ref)) of the state products. Elements at fidx(); the
// channels of each 32-group sit in kperm() order, the order in which the
// state's rows feed a product from registers (any order serves A and M).
// Double-buffered: the state waves read chunk i's while the helpers write
// chunk i+1's.
struct alignas(16) Fac {
    __bf16 Kah[ROWS32];             // k * exp(Gamma_r - Gamma_ref) = Kah + Kal
    __bf16 Kal[ROWS32];
    __bf16 Qah[ROWS32];             // q * exp(Gamma_r - Gamma_ref) = Qah + Qal
    __bf16 Qal[ROWS32];
    __bf16 Kbh[ROWS32];             // k * exp(Gamma_ref - Gamma_r) = Kbh + Kbl
    __bf16 Kbl[ROWS32];
};
// The part of Fac the state waves read (the two-kernel form carries it in its records).
constexpr int FAC_STATE_BYTES = 4 * ROWS32 * 2;

struct alignas(16) Smem {
    Ops op[2];
    Fac fac[2];
    // per helper wave: segment sums of each channel pair, segment s of pair cp
    // at s ^ (cp & 4), so that the 32 stores of a half-wave and the 16-byte
    // reads of segment pairs both meet distinct banks
    float2 segsum[NH][8][NSEG];
    int seq;                        // the sequence this workgroup runs (varlen)
};
static_assert(sizeof(Smem) <= 160 * 1024, "one workgroup per CU");

// x = hi + lo for a pair of floats: hi is x cut to bf16 (its upper 16 bits, so
// x - hi is exact), lo is that remainder rounded to bf16; together they carry
// about 16 significant bits.
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    const uint32_t u0 = __float_as_uint(x0), u1 = __float_as_uint(x1);
    hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);   // upper halves: x0 low word, x1 high word
    lo = pack_bf16(x0 - __uint_as_float(u0 & 0xffff0000u), x1 - __uint_as_float(u1 & 0xffff0000u));
}

__device__ __forceinline__ float2 bf2(uint32_t u) {
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}

// One helper lane's inputs of a chunk: channels 2cp, 2cp+1 (of its wave's 16)
// of tokens 4seg .. 4seg+3, and beta of one token. Tokens past the chunk's end
// read as zero (see chunk_rsrc), which makes their gate, key and query vanish
// from every product.
struct HFetch {
    float2 g[SEG];
    uint32_t k[SEG], q[SEG];
    float beta;
};
// Byte offsets of those elements within a chunk of k or q, of g, and of beta.
// With a scalar gate (SG) g has beta's layout and gg[t] is token t's offset there.
struct HOffs {
    uint32_t kq[SEG], gg[SEG], b;
    bool beta;                      // this wave stores beta (helper wave 0): only it loads it
};

// The fetch is split: k, q and beta (hfetch_kq) early in the element work, g
// (hfetch_g) at its end. Issuing the scattered loads stalls the issuing wave;
// the g loads, moved behind the element work, no longer hold up its segment-sum
// exchange (5% of the chunk period).
template <bool SG>
__device__ __forceinline__ void hfetch_kq(HFetch& f, const FwdArgs& a, long long cbase, long long cbeta,
                                          uint32_t ts, int nv, const HOffs& off) {
    const auto rk = chunk_rsrc(a.k, cbase, 2, nv, ts, D);
    const auto rq = chunk_rsrc(a.q, cbase, 2, nv, ts, D);
    const auto rb = chunk_rsrc(a.beta, cbeta, 4, nv, (uint32_t)a.H, 1);
#pragma unroll
    for (int t = 0; t < SEG; ++t) {
        f.k[t] = __builtin_amdgcn_raw_buffer_load_b32(rk, off.kq[t], 0, 0);
        f.q[t] = __builtin_amdgcn_raw_buffer_load_b32(rq, off.kq[t], 0, 0);
    }
    if (off.beta) f.beta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, off.b, 0, 0));
}
template <bool SG>
__device__ __forceinline__ void hfetch_g(HFetch& f, const FwdArgs& a, long long cbase, long long cbeta,
                                         uint32_t ts, int nv, const HOffs& off) {
    const auto rg = SG ? chunk_rsrc(a.g, cbeta, 4, nv, (uint32_t)a.H, 1) : chunk_rsrc(a.g, cbase, 4, nv, ts, D);
#pragma unroll
    for (int t = 0; t < SEG; ++t) {
        if constexpr (SG) {
            const float gs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, off.gg[t], 0, 0));
            f.g[t] = make_float2(gs, gs);
        } else {
            f.g[t] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(rg, off.gg[t], 0, 0));
        }
    }
}
template <bool SG>
__device__ __forceinline__ void hfetch(HFetch& f, const FwdArgs& a, long long cbase, long long cbeta,
                                       uint32_t ts, int nv, const HOffs& off) {
    hfetch_kq<SG>(f, a, cbase, cbeta, ts, nv, off);
    hfetch_g<SG>(f, a, cbase, cbeta, ts, nv, off);
}

// State waves: the lane's V column vc for a chunk's rows 16 (i >> 2) + 4 grp +
// (i & 3), i = 0..7, as raw bf16 bits in the low half (zero past the chunk's
// end). Lanes 2a and 2a + 1 (columns vc, vc + 1) load 4-byte column pairs,
// the even lane rows i = 0..3 and the odd lane rows i = 4..7: half the load
// instructions of 2-byte loads. voff2 holds those byte offsets (vpair_offsets);
// vunpack() trades the partner's half once the loads have landed.
__device__ __forceinline__ void vpair_offsets(uint32_t (&voff2)[4], int grp, int vc, uint32_t ts) {
    const int odd = vc & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) voff2[i] = ((uint32_t)(16 * odd + 4 * grp + i) * ts + (uint32_t)(vc & ~1)) * 2u;
}
__device__ __forceinline__ void vload(uint32_t (&raw)[4], __amdgpu_buffer_rsrc_t rv, const uint32_t (&voff2)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff2[i], 0, 0);
}
__device__ __forceinline__ void vunpack(uint32_t (&v)[8], const uint32_t (&raw)[4], int odd) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t p = (uint32_t)__builtin_amdgcn_mov_dpp((int)raw[i], 0xB1, 0xF, 0xF, false);   // lane l ^ 1
        v[i] = odd ? (p >> 16) : (raw[i] & 0xffffu);
        v[4 + i] = odd ? (raw[i] >> 16) : (p & 0xffffu);
    }
}

// A helper lane's gated keys and queries in fp32 and its channels' decay
// factors, kept in registers from step 1 to step 3.
struct HStage {
    float kb[2][SEG];                           // k e^(G_ref - G_r)
    float c1[2], c2[2];                         // e^(G_ref), e^(G_last - G_ref)
};

// Helpers, step 1: the gated factors of one chunk from the fetched registers,
// then the fetch of the chunk after it into the same registers.
//
// In-chunk cumulative log-gate Gamma, per channel, from the eight segment sums
// S0..S7 of 4-token segments. Every factor of A and M is referenced to
// Gamma_ref = Gamma at token 15 = S0+..+S3, so exponents stay within
// [-80, 75] for g in [-5, 0]: k*exp(Gamma_r - Gamma_ref) and
// k*exp(Gamma_ref - Gamma_i) multiply to k k exp(Gamma_r - Gamma_i) for every
// pair of tokens in the chunk. wpre holds this lane's weights of S0..S6 in
// Gamma at its segment start minus Gamma_ref (-1, 0 or +1).
template <bool SG>
__device__ __forceinline__ void factors(Smem& sm, Ops& op, Fac& fc, HFetch& f, HStage& hs, int hw, int lane,
                                        const float (&wpre)[NSEG - 1],
                                        bool fetch_next, const FwdArgs& a, long long nbase, long long nbeta,
                                        uint32_t ts, const HOffs& offs, int nnv) {
    const int cp = lane & 7, seg = lane >> 3;
    const int c0 = hchan(hw, cp);

    float L[2][SEG], kv[2][SEG], qv[2][SEG];
    float r0 = f.g[0].x, r1 = f.g[0].y;
#pragma unroll
    for (int t = 0; t < SEG; ++t) {
        if (t > 0) {
            r0 += f.g[t].x;
            r1 += f.g[t].y;
        }
        L[0][t] = r0;
        L[1][t] = r1;
        const float2 k2 = bf2(f.k[t]), q2 = bf2(f.q[t]);
        kv[0][t] = k2.x; kv[1][t] = k2.y;
        qv[0][t] = q2.x; qv[1][t] = q2.y;
    }
    sm.segsum[hw][cp][seg ^ (cp & 4)] = make_float2(r0, r1);   // see Smem::segsum
    if (hw == 0 && cp < SEG) op.beta[SEG * seg + cp] = f.beta;
    // The fp32 keys and queries are formed before the next chunk's loads are
    // issued, which frees the fetched registers for them. Left free, the
    // compiler sinks the conversions into the element loop; the new loads then
    // land in other registers, copied back at the end of the chunk behind a
    // wait for every outstanding load, the g prefetch included.
#pragma unroll
    for (int t = 0; t < SEG; ++t)
        asm volatile("" : "+v"(kv[0][t]), "+v"(kv[1][t]), "+v"(qv[0][t]), "+v"(qv[1][t]));
    // k, q and beta are consumed: fetch the chunk after this one (g follows
    // at the end, see hfetch_kq)
    if (fetch_next) hfetch_kq<SG>(f, a, nbase, nbeta, ts, nnv, offs);

    // all eight segment sums of this channel pair (written by this wave)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float St[2][NSEG];
#pragma unroll
    for (int s = 0; s < NSEG; s += 2) {
        const float4 v = lds_vec<float4>(&sm.segsum[hw][cp][s ^ (cp & 4)]);   // segments s, s + 1
        St[0][s] = v.x; St[1][s] = v.y; St[0][s + 1] = v.z; St[1][s + 1] = v.w;
    }
    float d[2][SEG];
    float (&c1)[2] = hs.c1;
    float (&c2)[2] = hs.c2;
    // A scalar gate gives both channels of the lane the same factors: form
    // them once (the same operations, so the values are the channel-wise ones).
    constexpr int NCH = SG ? 1 : 2;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const float* S = St[ch];
        const float ref = (S[0] + S[1]) + (S[2] + S[3]);
        const float last = (S[4] + S[5]) + (S[6] + S[7]);      // Gamma_last - Gamma_ref
        float moff = 0.f;
#pragma unroll
        for (int s = 0; s < NSEG - 1; ++s) moff = fmaf(wpre[s], S[s], moff);
        c1[ch] = ex2(ref * LOG2E);     // exp(Gamma_ref)              -> K*gamma, Q*gamma
        c2[ch] = ex2(last * LOG2E);    // exp(Gamma_last - Gamma_ref) -> Kt
        const float m2 = moff * LOG2E;
#pragma unroll
        for (int t = 0; t < SEG; ++t) d[ch][t] = fmaf(L[ch][t], LOG2E, m2);
    }
    if constexpr (SG) {
        c1[1] = c1[0];
        c2[1] = c2[0];
    }
    if (seg == 0) *reinterpret_cast<float2*>(&op.gl[c0]) = make_float2(c1[0] * c2[0], c1[1] * c2[1]);
    if (seg == 1) *reinterpret_cast<float2*>(&op.c1[c0]) = make_float2(c1[0], c1[1]);

    // channel position within the factor arrays' rows (kperm order per 32-group;
    // c0 is even, so the pair stays adjacent)
    const int cpos = (c0 & ~31) | kperm(c0 & 31);
#pragma unroll
    for (int t = 0; t < SEG; ++t) {
        const int so = fidx(SEG * seg + t, cpos);
        float ka[2][SEG], qa[2][SEG];
        float (&kb)[2][SEG] = hs.kb;
        float e1s[2], e2s[2];
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            e1s[ch] = ex2(d[ch][t]);
            e2s[ch] = ex2(-d[ch][t]);
        }
        if constexpr (SG) {
            e1s[1] = e1s[0];
            e2s[1] = e2s[0];
        }
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            const float e1 = e1s[ch], e2 = e2s[ch];
            ka[ch][t] = kv[ch][t] * e1;
            qa[ch][t] = qv[ch][t] * e1;
            kb[ch][t] = kv[ch][t] * e2;
        }
        uint32_t kah, kal, kbh, kbl, qah, qal;
        split_bf16x2(ka[0][t], ka[1][t], kah, kal);
        split_bf16x2(kb[0][t], kb[1][t], kbh, kbl);
        split_bf16x2(qa[0][t], qa[1][t], qah, qal);
        *reinterpret_cast<uint32_t*>(&fc.Kah[so]) = kah;
        *reinterpret_cast<uint32_t*>(&fc.Kal[so]) = kal;
        *reinterpret_cast<uint32_t*>(&fc.Kbh[so]) = kbh;
        *reinterpret_cast<uint32_t*>(&fc.Kbl[so]) = kbl;
        *reinterpret_cast<uint32_t*>(&fc.Qah[so]) = qah;
        *reinterpret_cast<uint32_t*>(&fc.Qal[so]) = qal;
    }
    if (fetch_next) hfetch_g<SG>(f, a, nbase, nbeta, ts, nnv, offs);
}

// The value x of lane l ^ 32 (v_permlane32_swap exchanges the upper half of
// its first operand with the lower half of its second; with both x, the lower
// lanes find their partners' x in the second result, the upper lanes in the
// first). No LDS traffic.
__device__ __forceinline__ uint32_t from_lane_xor32(uint32_t x, int upper) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return upper ? r[0] : r[1];
}

// Helpers, step 3: the state waves' fp16 operand K~^T of the lane's elements.
// Needed only from the next chunk on, so this VALU work runs after the
// mid-chunk barrier, beside the block products. Lanes l and l + 32 hold
// tokens 4s..4s+3 and 16+4s..16+4s+3 of the same two channels, the two halves
// of one 16-byte kperm piece: they trade one channel's half, and each stores
// one whole piece (lane l keeps channel cp & 1, lane l + 32 the other).
__device__ __forceinline__ void state_operands(Ops& op, const HStage& hs, int hw, int lane) {
    const int cp = lane & 7, seg = lane >> 3;
    const int c0 = hchan(hw, cp);
    uint2 pk[2];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        const float c2 = hs.c2[ch];
        pk[ch] = make_uint2(pack_f16(hs.kb[ch][0] * c2, hs.kb[ch][1] * c2), pack_f16(hs.kb[ch][2] * c2, hs.kb[ch][3] * c2));
    }
    const int upper = seg >> 2;                 // lanes 32-63: tokens 16-31
    const int keep = (cp & 1) ^ upper;          // the channel this lane stores
    const uint2 send = keep ? pk[0] : pk[1];
    const uint2 mine = keep ? pk[1] : pk[0];
    const uint2 got = make_uint2(from_lane_xor32(send.x, upper), from_lane_xor32(send.y, upper));
    const uint4 piece = upper ? make_uint4(got.x, got.y, mine.x, mine.y) : make_uint4(mine.x, mine.y, got.x, got.y);
    const int row = c0 + keep;
    *reinterpret_cast<uint4*>(&op.KtT[row][kcol(row, 8 * (seg & 3))]) = piece;
}

// X Y for 16 x 16 matrices, from X^T and Y in accumulator layout (lane: rows
// 4grp+j, column l16), into the same layout, added to c (fp32). That layout is
// both the A operand of X (row l16, K-slots 4grp+j) and the B operand of Y
// (K-slots 4grp+j, column l16) of one 16x16x16 fp16 MFMA: the operands are
// rounded to fp16, the product accumulates in fp32.
__device__ __forceinline__ f32x4 mprod(const f32x4& xt, const f32x4& y, f32x4 c) {
    const f16x4 a = {(_Float16)xt[0], (_Float16)xt[1], (_Float16)xt[2], (_Float16)xt[3]};
    const f16x4 b = {(_Float16)y[0], (_Float16)y[1], (_Float16)y[2], (_Float16)y[3]};
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Stores a 16 x 16 accumulator tile (lane: rows 4grp+j, column l16) into a
// [row][kperm(col)] fp16 array as 32-bit pairs of adjacent columns: the two
// lanes of a column pair swap half their rows, so an even lane writes rows j
// = 0, 2 and an odd lane rows 1, 3. With two arrays (hi, lo) the value is
// stored as a two-term split. Diagonal tiles keep col <= row.
template <bool SPLIT>
__device__ __forceinline__ void store_tile(_Float16 (*hi)[TP], _Float16 (*lo)[TP], const f32x4& m, int r0, int c0,
                                           bool diag, int l16, int grp) {
    const bool odd = l16 & 1;
    float mine[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * grp + j;
        mine[j] = (!diag || l16 <= r) ? m[j] : 0.f;
    }
    // send the rows the partner writes: even lanes send rows 1, 3; odd lanes rows 0, 2
    const float got0 = swap_pair(odd ? mine[0] : mine[1]);
    const float got1 = swap_pair(odd ? mine[2] : mine[3]);
    const int cpos = kperm(c0 + (l16 & ~1));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int j = 2 * h + (odd ? 1 : 0);
        const float own = odd ? (h ? mine[3] : mine[1]) : (h ? mine[2] : mine[0]);
        const float oth = h ? got1 : got0;
        const float x0 = odd ? oth : own, x1 = odd ? own : oth;   // columns c0 + 2a, c0 + 2a + 1
        const int r = r0 + 4 * grp + j;
        if constexpr (SPLIT) {
            uint32_t wh, wl;
            split_f16x2(x0, x1, wh, wl);
            *reinterpret_cast<uint32_t*>(&hi[r][tcol(r, cpos)]) = wh;
            *reinterpret_cast<uint32_t*>(&lo[r][tcol(r, cpos)]) = wl;
        } else {
            *reinterpret_cast<uint32_t*>(&hi[r][tcol(r, cpos)]) = pack_f16(x0, x1);
        }
    }
}

// (I + A_bb)^{-1} of one diagonal block, from A_bb in fp32 (op.Af), into Tm as
// an fp16 operand. (I + A)^{-1} = (I - A)(I + A^2)(I + A^4)(I + A^8): A
// is strictly lower triangular, so A^16 = 0 and the product is the whole
// Neumann series (the factors commute). The identity terms stay exact in the
// fp32 accumulators; only the powers of A pass through fp16 operands. With
// |A_ri| <= about 1 (unit keys, beta <= 1, decays <= 1) an entry of A^n is at
// most C(14, n-1), so A^8 stays below 3432, well inside fp16's range.
__device__ __forceinline__ void invert_block(Ops& op, int b, int l16, int grp) {
    f32x4 A, At, ImA;
    const float4 t4 = lds_vec<float4>(&op.Af[b][l16][4 * grp]);   // A^T in accumulator layout
    At[0] = t4.x; At[1] = t4.y; At[2] = t4.z; At[3] = t4.w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 4 * grp + j;
        A[j] = op.Af[b][r][l16];
        ImA[j] = (l16 == r ? 1.f : 0.f) - A[j];
    }
    const f32x4 Z = {0.f, 0.f, 0.f, 0.f};
    const f32x4 A2 = mprod(At, A, Z), A2t = mprod(A, At, Z);
    const f32x4 Q1 = mprod(A2t, ImA, ImA);               // (I + A^2)(I - A)
    const f32x4 A4 = mprod(A2t, A2, Z), A4t = mprod(A2, A2t, Z);
    const f32x4 Q2 = mprod(A4t, Q1, Q1);                 // (I + A^4) Q1
    const f32x4 A8t = mprod(A4, A4t, Z);
    const f32x4 Tb = mprod(A8t, Q2, Q2);                 // (I + A^8) Q2
    store_tile<false>(op.Tm, nullptr, Tb, 16 * b, 16 * b, false, l16, grp);
}

// Helpers, step 2: the gated K K^T blocks of A and the gated Q K^T blocks of
// M, each from two-term bf16 factors (three MFMA terms), fp32 accumulation:
//   block 0 A00, 1 A11, 2 A10, 3 M00, 4 M10, 5 M11.
// A00 and A11 go to the state waves in fp32 (they invert I + A there, under
// the helpers' element work); A10 and M are stored as fp16 operands. The zero
// blocks of Tm, A10 and M are written once, at the kernel's start. The wave
// forms its K~^T pieces under the block's products.
__device__ __forceinline__ void tile_block(const Fac& fc, Ops& op, const HStage& hs, int hw, int lane, int blk) {
    const int l16 = lane & 15, grp = lane >> 4;
    if (blk <= 2) {
        // A[r][i] = beta_r (Ka_r . Kb_i) = beta_r (Kah Kbh + Kah Kbl + Kal Kbh):
        // lane holds column i = l16 of rows r = 4grp + j
        const int rb = blk == 0 ? 0 : 16, cb = blk == 1 ? 16 : 0;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc1 = acc, acc2 = acc;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            const int ko = 32 * kk + 8 * grp;
            const bf16x8 kah = lds_vec<bf16x8>(&fc.Kah[fidx(rb + l16, ko)]);
            const bf16x8 kal = lds_vec<bf16x8>(&fc.Kal[fidx(rb + l16, ko)]);
            const bf16x8 kbh = lds_vec<bf16x8>(&fc.Kbh[fidx(cb + l16, ko)]);
            const bf16x8 kbl = lds_vec<bf16x8>(&fc.Kbl[fidx(cb + l16, ko)]);
            acc = mfma16(kah, kbh, acc);
            acc1 = mfma16(kah, kbl, acc1);
            acc2 = mfma16(kal, kbh, acc2);
        }
        state_operands(op, hs, hw, lane);   // VALU work while the products finish
        acc += acc1 + acc2;
        if (blk < 2) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * grp + j;
                op.Af[blk][r][l16] = (l16 < r) ? op.beta[rb + r] * acc[j] : 0.f;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] *= op.beta[16 + 4 * grp + j];
            store_tile<false>(op.A10, nullptr, acc, 0, 0, false, l16, grp);
        }
    } else {
        // M[r][i] = Qa_r . Kb_i (i <= r) = Qah Kbh + Qah Kbl + Qal Kbh
        const int rb = blk == 3 ? 0 : 16, cb = blk == 5 ? 16 : 0;
        f32x4 m0 = {0.f, 0.f, 0.f, 0.f}, m1 = m0, m2 = m0;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            const int ko = 32 * kk + 8 * grp;
            const bf16x8 qh = lds_vec<bf16x8>(&fc.Qah[fidx(rb + l16, ko)]);
            const bf16x8 ql = lds_vec<bf16x8>(&fc.Qal[fidx(rb + l16, ko)]);
            const bf16x8 kh = lds_vec<bf16x8>(&fc.Kbh[fidx(cb + l16, ko)]);
            const bf16x8 kl = lds_vec<bf16x8>(&fc.Kbl[fidx(cb + l16, ko)]);
            m0 = mfma16(qh, kh, m0);
            m1 = mfma16(qh, kl, m1);
            m2 = mfma16(ql, kh, m2);
        }
        state_operands(op, hs, hw, lane);
        store_tile<true>(op.M[0], op.M[1], m0 + (m1 + m2), rb, cb, blk != 4, l16, grp);
    }
}

// The block of helper wave hw with NS state waves (0xFF: none). The waves of
// a workgroup go to the four SIMDs in turn, so waves w and w + 4 share one
// (helper hw is wave NS + hw); one block per wave keeps the helpers' second
// phase short.
//   NS = 4: every SIMD holds a state wave, and SIMDs 0 and 1 also run the
//           inverses: one block each there, two each on the other two;
//   NS = 8: the same with two state waves per SIMD;
//   NS = 2: two blocks on each of the two SIMDs without a state wave, one on
//           each of the others;
//   NS = 1: one block on each helper wave of the three SIMDs without the state wave.
// The table's bytes are shifted out with scalar instructions: a table in
// memory would be a load, and its wait inside the chunk loop would also wait
// for the input prefetch.
template <int NS>
__device__ __forceinline__ int helper_block(int hw) {
    constexpr uint64_t T = (NS == 4 || NS == 8) ? 0x0504FFFF03020100ull : (NS == 2 ? 0xFFFF050304020100ull : 0xFF050301FF040200ull);
    return (int)((T >> (8 * hw)) & 0xFFu);
}

template <int NS>
__device__ __forceinline__ void tiles(const Fac& fc, Ops& op, const HStage& hs, int hw, int lane) {
    const int blk = helper_block<NS>(hw);
    if (blk == 0xFF) state_operands(op, hs, hw, lane);
    else tile_block(fc, op, hs, hw, lane, blk);
}

// State waves, first step of a chunk: P = (K*gamma) S and O1 = (Q*gamma) S
// for the wave's 16 columns, as Ka (Diag(e^Gamma_ref) S) and Qa (Diag(e^Gamma_ref) S)
// with every operand two-term bf16 (three MFMA terms each): the scaled state
// as a B operand with its rows in kperm order, the factors as A operands.
// `fc` holds Kah, Kal, Qah, Qal of the chunk (only those members are read).
template <typename F>
__device__ __forceinline__ void state_products(const f32x4 (&S)[8], const Ops& op, const F& fc, int l16, int grp,
                                               f32x4 (&Pt)[2], f32x4 (&Ot)[2]) {
    bf16x8 SBh[4], SBl[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        // rows 32kk + 4grp + j (slots 0-3) and 32kk + 16 + 4grp + j (slots 4-7)
        const float4 ca = lds_vec<float4>(&op.c1[32 * kk + 4 * grp]);
        const float4 cb = lds_vec<float4>(&op.c1[32 * kk + 16 + 4 * grp]);
        uint32_t h[4], l[4];
        split_bf16x2(S[2 * kk][0] * ca.x, S[2 * kk][1] * ca.y, h[0], l[0]);
        split_bf16x2(S[2 * kk][2] * ca.z, S[2 * kk][3] * ca.w, h[1], l[1]);
        split_bf16x2(S[2 * kk + 1][0] * cb.x, S[2 * kk + 1][1] * cb.y, h[2], l[2]);
        split_bf16x2(S[2 * kk + 1][2] * cb.z, S[2 * kk + 1][3] * cb.w, h[3], l[3]);
        SBh[kk] = __builtin_bit_cast(bf16x8, h);
        SBl[kk] = __builtin_bit_cast(bf16x8, l);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        Pt[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        Ot[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int off = fidx(16 * t + l16, 32 * kk + 8 * grp);
            const bf16x8 kh = lds_vec<bf16x8>(&fc.Kah[off]), kl = lds_vec<bf16x8>(&fc.Kal[off]);
            const bf16x8 qh = lds_vec<bf16x8>(&fc.Qah[off]), ql = lds_vec<bf16x8>(&fc.Qal[off]);
            Pt[t] = mfma16(kh, SBh[kk], Pt[t]);
            Ot[t] = mfma16(qh, SBh[kk], Ot[t]);
            Pt[t] = mfma16(kh, SBl[kk], Pt[t]);
            Ot[t] = mfma16(qh, SBl[kk], Ot[t]);
            Pt[t] = mfma16(kl, SBh[kk], Pt[t]);
            Ot[t] = mfma16(ql, SBh[kk], Ot[t]);
        }
    }
}

// State waves, second step of a chunk (after the mid-chunk barrier): the
// solve Delta = (I + A)^{-1} Diag(beta) (V - P) over the two diagonal blocks,
// the output O = O1 + M Delta stored through `ro`, and the state update
// S <- Diag(gamma_last) S + Kt^T Delta. bt0, bt1 (beta) and a10 (A10) were read
// before the barrier; vcur holds V of the wave's column (raw bf16 bits).
__device__ __forceinline__ void state_finish(f32x4 (&S)[8], const Ops& op, const f32x4 (&Pt)[2], const f32x4 (&Ot)[2],
                                             const uint32_t (&vcur)[8], const float4& bt0, const float4& bt1,
                                             const f16x4& a10, __amdgpu_buffer_rsrc_t ro, const uint32_t (&voff)[8],
                                             int l16, int grp) {
    const float bts[2][4] = {{bt0.x, bt0.y, bt0.z, bt0.w}, {bt1.x, bt1.y, bt1.z, bt1.w}};
    float be[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            be[t][j] = bts[t][j] * (__uint_as_float(vcur[4 * t + j] << 16) - Pt[t][j]);
    // The solve runs on 16x16x16 MFMAs: the A operand is the half of a row's
    // 16-byte kperm piece that holds the block's columns 4grp..4grp+3, the B
    // operand four halves (tokens 4grp+j of one sub-block, column l16).
    // Delta0 = T00 bE0 (two-term fp16 operand)
    const f32x4 Z = {0.f, 0.f, 0.f, 0.f};
    uint32_t bh[2], bl[2];
    split_f16x2(be[0][0], be[0][1], bh[0], bl[0]);
    split_f16x2(be[0][2], be[0][3], bh[1], bl[1]);
    const f16x4 t00 = lds_vec<f16x4>(&op.Tm[l16][tcol(l16, 8 * grp)]);
    f32x4 D0 = __builtin_amdgcn_mfma_f32_16x16x16f16(t00, __builtin_bit_cast(f16x4, bh), Z, 0, 0, 0);
    D0 = __builtin_amdgcn_mfma_f32_16x16x16f16(t00, __builtin_bit_cast(f16x4, bl), D0, 0, 0, 0);
    uint32_t dh[4], dl[4];
    split_f16x2(D0[0], D0[1], dh[0], dl[0]);
    split_f16x2(D0[2], D0[3], dh[1], dl[1]);
    // Delta1 = T11 (bE1 - A10 Delta0)
    const uint2 d0h = make_uint2(dh[0], dh[1]), d0l = make_uint2(dl[0], dl[1]);
    f32x4 X = __builtin_amdgcn_mfma_f32_16x16x16f16(a10, __builtin_bit_cast(f16x4, d0h), Z, 0, 0, 0);
    X = __builtin_amdgcn_mfma_f32_16x16x16f16(a10, __builtin_bit_cast(f16x4, d0l), X, 0, 0, 0);
    split_f16x2(be[1][0] - X[0], be[1][1] - X[1], bh[0], bl[0]);
    split_f16x2(be[1][2] - X[2], be[1][3] - X[3], bh[1], bl[1]);
    const f16x4 t11 = lds_vec<f16x4>(&op.Tm[16 + l16][tcol(l16, 8 * grp) + 4]);
    f32x4 D1 = __builtin_amdgcn_mfma_f32_16x16x16f16(t11, __builtin_bit_cast(f16x4, bh), Z, 0, 0, 0);
    D1 = __builtin_amdgcn_mfma_f32_16x16x16f16(t11, __builtin_bit_cast(f16x4, bl), D1, 0, 0, 0);
    split_f16x2(D1[0], D1[1], dh[2], dl[2]);
    split_f16x2(D1[2], D1[3], dh[3], dl[3]);
    const f16x8 DBh = __builtin_bit_cast(f16x8, dh), DBl = __builtin_bit_cast(f16x8, dl);
    // O = (Q*gamma) S + M Delta (rows past the chunk's end are dropped)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const f16x8 mh = lds_vec<f16x8>(&op.M[0][16 * t + l16][tcol(l16, 8 * grp)]);
        const f16x8 ml = lds_vec<f16x8>(&op.M[1][16 * t + l16][tcol(l16, 8 * grp)]);
        f32x4 acc = Ot[t];
        acc = mfma16(mh, DBh, acc);
        acc = mfma16(mh, DBl, acc);
        acc = mfma16(ml, DBh, acc);
        const float ov[4] = {acc[0], acc[1], acc[2], acc[3]};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov[j]), ro, 2u * voff[4 * t + j], 0, 0);
    }
    // S <- Diag(gamma_last) S + Kt^T Delta (single fp16 Kt, two-term Delta)
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float4 g4 = lds_vec<float4>(&op.gl[16 * m + 4 * grp]);
        S[m][0] *= g4.x;
        S[m][1] *= g4.y;
        S[m][2] *= g4.z;
        S[m][3] *= g4.w;
        const f16x8 kt = lds_vec<f16x8>(&op.KtT[16 * m + l16][kcol(16 * m + l16, 8 * grp)]);
        S[m] = mfma16(kt, DBh, S[m]);
        S[m] = mfma16(kt, DBl, S[m]);
    }
}

template <int NS, bool SG>
__global__ __launch_bounds__(64 * (NS + NH), 1) void kda_fwd_pipe(FwdArgs a) {
    constexpr int NT = Split<NS>::NT, VB = Split<NS>::VB, P = Split<NS>::P;
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave: scalar branches on roles
    const int l16 = lane & 15, grp = lane >> 4;
    const bool is_state = wave < NS;

    // The P V-blocks of a (sequence, head) sit eight workgroups apart, so they
    // land on the same XCD and share its L2 for q, k and g.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, rest = bid >> 3;
    const int vblk = rest % P;
    const int chain = (rest / P) * 8 + xcd;
    if (chain >= a.nchains) return;
    const int NH_ = a.N * a.H;
    const int task = a.ntasks > 0 ? chain / NH_ : 0;
    const int h = chain % a.H;
    int n = (chain % NH_) / a.H;
    if (a.cu && a.N <= MAX_RANKED) {
        // Longest sequences first: workgroups are dispatched roughly in id
        // order, so the long chains start early and the short ones fill in
        // behind them. Sequence rank = number of longer ones (ties by index).
        if (tid < a.N) {
            const int len = a.cu[tid + 1] - a.cu[tid];
            int rank = 0;
            for (int m = 0; m < a.N; ++m) {
                const int lm = a.cu[m + 1] - a.cu[m];
                rank += (lm > len || (lm == len && m < tid)) ? 1 : 0;
            }
            if (rank == n) sm.seq = tid;
        }
        __syncthreads();
        n = __builtin_amdgcn_readfirstlane(sm.seq);
    }
    int row, t0, t1;
    const float* h0p = a.h0;
    float* hTp = a.hT;
    float* outp = a.o;              // o of this workgroup's task, token 0 at token ot0 of the row
    int ot0 = 0, oT = a.T;
    int tflags = 0;
    if (a.cu) { row = 0; t0 = a.cu[n]; t1 = a.cu[n + 1]; }
    else      { row = n; t0 = 0;       t1 = a.T; }
    if (a.ntasks > 0) {
        // The task index is uniform, but a dynamic index into the argument
        // block is not seen as such: make the fields scalar again, or every
        // buffer resource built from them would need a waterfall loop.
        const FwdTask& tk = a.task[task];
        t0 = __builtin_amdgcn_readfirstlane(tk.t_begin);
        t1 = __builtin_amdgcn_readfirstlane(tk.t_end);
        tflags = __builtin_amdgcn_readfirstlane(tk.flags);
        const auto uptr = [](const void* p) {
            const uint64_t u = reinterpret_cast<uint64_t>(p);
            const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
            const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
            return ((uint64_t)hi << 32) | lo;
        };
        h0p = reinterpret_cast<const float*>(uptr(tk.h0));
        hTp = reinterpret_cast<float*>(uptr(tk.hT));
        float* to = reinterpret_cast<float*>(uptr(tk.o));
        if (to) {
            outp = to;
            ot0 = __builtin_amdgcn_readfirstlane(tk.o_t0);
            oT = __builtin_amdgcn_readfirstlane(tk.o_T);
        }
    }
    // uniform per workgroup: keep them scalar (buffer resources are built from them)
    t0 = __builtin_amdgcn_readfirstlane(t0);
    t1 = __builtin_amdgcn_readfirstlane(t1);
    const int nch = (t1 - t0 + C - 1) / C;
    const uint32_t ts = (uint32_t)a.H * D;
    const long long base = (long long)row * a.T * ts + (long long)h * D;
    const long long bbase = (long long)row * a.T * a.H + h;
    const long long sbase = ((long long)n * a.H + h) * D * D;
    const long long obase = ((long long)row * oT - ot0) * ts + (long long)h * D;   // o of token 0 (from token ot0 on)

    // Zero blocks of both operand buffers, never written afterwards: kperm
    // positions 16-31 of rows 0-15 in Tm, M (hi, lo) and A10, and positions
    // 0-15 of rows 16-31 in Tm.
    for (int i = tid; i < 2 * C * 8; i += NT) {
        const int bsel = i / (C * 8), r = (i / 8) % C, c = 2 * (i % 8);
        const int col = kperm((r < 16 ? 16 : 0) + c);
        Ops& op = sm.op[bsel];
        *reinterpret_cast<uint32_t*>(&op.Tm[r][tcol(r, col)]) = 0u;
        if (r < 16) {
            *reinterpret_cast<uint32_t*>(&op.M[0][r][tcol(r, col)]) = 0u;
            *reinterpret_cast<uint32_t*>(&op.M[1][r][tcol(r, col)]) = 0u;
            *reinterpret_cast<uint32_t*>(&op.A10[r][tcol(r, col)]) = 0u;
        }
    }
    __syncthreads();

    // Both roles execute the same number of workgroup barriers: two or three
    // before the chunk loop and two per chunk.
    if (is_state) {
        const int vc = vblk * VB + wave * 16 + l16;                     // this lane's V column
        // byte offsets of (row 16t + 4grp + j, column vc) within a chunk of v (bf16)
        uint32_t voff[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) voff[i] = ((uint32_t)(16 * (i >> 2) + 4 * grp + (i & 3)) * ts + vc) * 2u;
        uint32_t voff2[4];
        vpair_offsets(voff2, grp, vc, ts);
        f32x4 S[8];
        uint32_t vcur[8], vraw[4];
        // V of this lane's column for the chunk's tokens 16t + 4grp + j (see vload)
        auto vfetch = [&](uint32_t (&dst)[4], int cidx) {
            const int cs = t0 + cidx * C;
            // an empty resource reads zeros (a slice run with v = 0)
            const auto rv = chunk_rsrc(a.v, base + (long long)cs * ts, 2, (tflags & TASK_ZERO_V) ? 0 : min(C, t1 - cs), ts, D);
            vload(dst, rv, voff2);
        };
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                S[m][j] = (tflags & TASK_IDENTITY_H0) ? (16 * m + 4 * grp + j == vc ? 1.f : 0.f)
                          : h0p ? h0p[sbase + (uint32_t)(16 * m + 4 * grp + j) * D + vc] : 0.f;
        // Complete the h0 loads here (s_waitcnt vmcnt(0)): otherwise the
        // compiler cannot prove them done inside the chunk loop and waits there
        // for every outstanding load, including the next chunk's prefetch.
        __builtin_amdgcn_s_waitcnt(0x0F70);
        // The state waves' dependent chain (solve, output, state update) sets
        // the length of each chunk's second phase, while the helpers have slack
        // there: the state waves issue first when both are ready.
        __builtin_amdgcn_s_setprio(2);
        if (nch > 0) {
            vfetch(vraw, 0);
            vunpack(vcur, vraw, vc & 1);
            __syncthreads();   // the helpers' mid-chunk barrier of chunk 0
        }
        __syncthreads();
        for (int ci = 0; ci < nch; ++ci) {
            const int cs = t0 + ci * C;
            const int nv = min(C, t1 - cs);
            Ops& opw = sm.op[ci & 1];
            const Ops& op = opw;
            // V of the next chunk, copied into vcur at the end of this one: the
            // loaded registers never stay pending across the loop edge, so the
            // waits for them are exact and fall after this chunk's work.
            if (ci + 1 < nch) vfetch(vraw, ci + 1);
            // (I + A)^{-1} of the two diagonal blocks, from the helpers' A of this
            // chunk, for all state waves after the mid-chunk barrier. It runs on
            // the matrix cores while the helpers' element work runs on the VALUs.
            if (NS == 1) {
                invert_block(opw, 0, l16, grp);
                invert_block(opw, 1, l16, grp);
            } else if (wave < 2) {
                invert_block(opw, wave, l16, grp);
            }
            f32x4 Pt[2], Ot[2];
            state_products(S, op, sm.fac[ci & 1], l16, grp, Pt, Ot);
            // beta and A10 of this chunk were written before the last barrier:
            // read them now, so the solve after the barrier starts without an
            // LDS round trip (T is written in this phase and is read after it).
            const float4 bt0 = lds_vec<float4>(&op.beta[4 * grp]), bt1 = lds_vec<float4>(&op.beta[16 + 4 * grp]);
            const f16x4 ah = lds_vec<f16x4>(&op.A10[l16][tcol(l16, 8 * grp)]);   // A10 row l16, columns 4grp..4grp+3
            __syncthreads();   // mid-chunk: the helpers' factors of chunk ci+1 are written
            // O's rows past the chunk's end are dropped; an empty resource drops
            // every store (a slice run for its state only)
            const auto ro = chunk_rsrc(outp, obase + (long long)cs * ts, 4, (tflags & TASK_NO_OUTPUT) ? 0 : nv, ts, D);
            state_finish(S, op, Pt, Ot, vcur, bt0, bt1, ah, ro, voff, l16, grp);
            vunpack(vcur, vraw, vc & 1);
            __syncthreads();
        }
        if (hTp) {
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    hTp[sbase + (uint32_t)(16 * m + 4 * grp + j) * D + vc] = S[m][j];
        }
    } else {
        const int hw = wave - NS;
        const int cp = lane & 7, seg = lane >> 3;
        const uint32_t coff = hchan(hw, cp);                           // channel pair offset
        // weights of the segment sums S0..S6 in Gamma(segment start) - Gamma_ref
        float wpre[NSEG - 1];
#pragma unroll
        for (int s = 0; s < NSEG - 1; ++s)
            wpre[s] = (s >= seg && s < NSEG / 2) ? -1.f : ((s >= NSEG / 2 && s < seg) ? 1.f : 0.f);
        HOffs offs;
#pragma unroll
        for (int t = 0; t < SEG; ++t) {
            offs.kq[t] = ((uint32_t)(SEG * seg + t) * ts + coff) * 2u;
            offs.gg[t] = SG ? (uint32_t)(SEG * seg + t) * (uint32_t)a.H * 4u : 2u * offs.kq[t];
        }
        offs.b = (uint32_t)(SEG * seg + (cp & 3)) * (uint32_t)a.H * 4u;
        offs.beta = hw == 0;
        HFetch f;
        HStage hs;
        auto prepare = [&](int buf, int cs) {
            const bool more = cs + C < t1;
            const int nnv = more ? min(C, t1 - cs - C) : 0;
            factors<SG>(sm, sm.op[buf], sm.fac[buf], f, hs, hw, lane, wpre, more, a, base + (long long)(cs + C) * ts,
                        bbase + (long long)(cs + C) * a.H, ts, offs, nnv);
            __syncthreads();   // mid-chunk barrier
            tiles<NS>(sm.fac[buf], sm.op[buf], hs, hw, lane);
        };
        if (nch > 0) {
            hfetch<SG>(f, a, base + (long long)t0 * ts, bbase + (long long)t0 * a.H, ts, min(C, t1 - t0), offs);
            prepare(0, t0);
        }
        __syncthreads();
        for (int ci = 0; ci < nch; ++ci) {
            // registers of chunk ci+1 were fetched during the previous prepare()
            if (ci + 1 < nch) prepare((ci + 1) & 1, t0 + (ci + 1) * C);
            else __syncthreads();   // the mid-chunk barrier of the last chunk
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// The same work as two kernels, the split the pages credit to FlashKDA (a
// chunk-parallel preparation, then the sequential recurrence; toolarium.ru
// page, section "Где ограничения прямо сейчас"), kept as an ablation of the
// kernel count. The preparation writes every chunk's Ops to HBM and the
// recurrence reads it back, so the arithmetic is the fused kernel's, value
// for value; only the place where the operands wait between the halves moves
// from LDS to HBM (1.28 KB more traffic per token-head each way).

// A record: the chunk's Ops and the four factor arrays of its state products.
struct alignas(16) RecOps {
    Ops op;
    __bf16 Kah[ROWS32], Kal[ROWS32], Qah[ROWS32], Qal[ROWS32];
};
static_assert(sizeof(RecOps) == sizeof(Ops) + FAC_STATE_BYTES, "no padding inside a record");
static_assert(sizeof(Ops) % 16 == 0 && FAC_STATE_BYTES % 16 == 0, "records are copied in 16-byte pieces");
constexpr int OPS_VEC = (int)(sizeof(RecOps) / 16);   // 16-byte pieces per record
// Copy waves of the recurrence kernel, and the record layout they move.
constexpr int NCW = 4;
constexpr int CG_LANES = 64 * (NCW / 2);                            // lanes of one copy group
constexpr int CG_REGS = (OPS_VEC + CG_LANES - 1) / CG_LANES;        // 16-byte pieces per copy lane
// Records are padded to a whole number of pieces per copy lane, so the copy
// loops need no per-piece bounds (which would put each load in its own branch
// and make the compiler wait for it there). The pad is never read.
constexpr int REC_PIECES = CG_REGS * CG_LANES;
struct alignas(16) OpsBuf {
    RecOps rec;
    uint4 pad[REC_PIECES - OPS_VEC];
};
static_assert(sizeof(OpsBuf) == 16 * REC_PIECES, "one record per operand buffer");

// A copy lane's pieces of one record: src[0], src[CG_LANES], ... (global), and
// the same positions of an operand buffer (LDS). Native vectors, so the
// pieces stay in registers.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void rec_load(u32x4 (&r)[CG_REGS], const u32x4* src) {
#pragma unroll
    for (int k = 0; k < CG_REGS; ++k) r[k] = src[CG_LANES * k];
}
__device__ __forceinline__ void rec_store(const u32x4 (&r)[CG_REGS], u32x4* dst) {
#pragma unroll
    for (int k = 0; k < CG_REGS; ++k) dst[CG_LANES * k] = r[k];
}

// Workgroups of the preparation: chunks [g * per_wg, (g + 1) * per_wg) of one
// (sequence, head), eight helper waves, fixed-length batches.
__global__ __launch_bounds__(64 * NH, 1) void kda_prep_pipe(FwdArgs a, uint4* rec, int nch, int per_wg) {
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int hw = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, grp = lane >> 4;
    const int ngrp = (nch + per_wg - 1) / per_wg;
    const int chain = blockIdx.x / ngrp;
    if (chain >= a.nchains) return;
    const int c_begin = (blockIdx.x % ngrp) * per_wg;
    const int c_end = min(nch, c_begin + per_wg);
    const int n = chain / a.H, h = chain % a.H;
    const int t0 = 0, t1 = a.T;
    const uint32_t ts = (uint32_t)a.H * D;
    const long long base = (long long)n * a.T * ts + (long long)h * D;
    const long long bbase = (long long)n * a.T * a.H + h;

    // the never-written zero blocks of both operand buffers (as in the fused kernel)
    for (int i = tid; i < 2 * C * 8; i += 64 * NH) {
        const int bsel = i / (C * 8), r = (i / 8) % C, c = 2 * (i % 8);
        const int col = kperm((r < 16 ? 16 : 0) + c);
        Ops& op = sm.op[bsel];
        *reinterpret_cast<uint32_t*>(&op.Tm[r][tcol(r, col)]) = 0u;
        if (r < 16) {
            *reinterpret_cast<uint32_t*>(&op.M[0][r][tcol(r, col)]) = 0u;
            *reinterpret_cast<uint32_t*>(&op.M[1][r][tcol(r, col)]) = 0u;
            *reinterpret_cast<uint32_t*>(&op.A10[r][tcol(r, col)]) = 0u;
        }
    }
    const int cp = lane & 7, seg = lane >> 3;
    const uint32_t coff = hchan(hw, cp);
    float wpre[NSEG - 1];
#pragma unroll
    for (int s = 0; s < NSEG - 1; ++s)
        wpre[s] = (s >= seg && s < NSEG / 2) ? -1.f : ((s >= NSEG / 2 && s < seg) ? 1.f : 0.f);
    HOffs offs;
#pragma unroll
    for (int t = 0; t < SEG; ++t) {
        offs.kq[t] = ((uint32_t)(SEG * seg + t) * ts + coff) * 2u;
        offs.gg[t] = 2u * offs.kq[t];
    }
    offs.b = (uint32_t)(SEG * seg + (cp & 3)) * (uint32_t)a.H * 4u;
    offs.beta = hw == 0;
    HFetch f;
    HStage hs;
    __syncthreads();
    if (c_begin < c_end) {
        const int cs = t0 + c_begin * C;
        hfetch<false>(f, a, base + (long long)cs * ts, bbase + (long long)cs * a.H, ts, min(C, t1 - cs), offs);
    }
    for (int ci = c_begin; ci < c_end; ++ci) {
        Ops& op = sm.op[ci & 1];
        Fac& fc = sm.fac[ci & 1];
        const int cs = t0 + ci * C;
        const bool more = ci + 1 < c_end;
        const int nnv = more ? min(C, t1 - cs - C) : 0;
        factors<false>(sm, op, fc, f, hs, hw, lane, wpre, more, a, base + (long long)(cs + C) * ts,
                       bbase + (long long)(cs + C) * a.H, ts, offs, nnv);
        __syncthreads();
        tiles<4>(fc, op, hs, hw, lane);   // eight helper waves, two per SIMD
        __syncthreads();
        if (hw < 2) invert_block(op, hw, l16, grp);
        __syncthreads();
        // the record: Ops, then Kah, Kal, Qah, Qal (the first four arrays of Fac)
        const uint4* src_op = reinterpret_cast<const uint4*>(&op);
        const uint4* src_fac = reinterpret_cast<const uint4*>(&fc);
        constexpr int OP_PIECES = (int)(sizeof(Ops) / 16);
        uint4* dst = rec + ((size_t)chain * nch + ci) * REC_PIECES;
        for (int i = tid; i < OPS_VEC; i += 64 * NH) dst[i] = i < OP_PIECES ? src_op[i] : src_fac[i - OP_PIECES];
    }
}

// The recurrence: NS state waves as in the fused kernel (the inverses now come
// with the record), and NCW copy waves that write chunk i+1's record into the
// other operand buffer while the state waves advance chunk i. One workgroup
// barrier per chunk.

// One workgroup per CU is the target (its LDS would allow two): the copy lanes
// hold a whole record piece set in registers.
template <int NS>
__global__ __launch_bounds__(64 * (NS + NCW), 1) __attribute__((amdgpu_waves_per_eu(1, 2)))
void kda_recur_pipe(FwdArgs a, const uint4* rec, int nch) {
    constexpr int VB = Split<NS>::VB, P = Split<NS>::P;
    __shared__ OpsBuf ops[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, grp = lane >> 4;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, rest = bid >> 3;
    const int vblk = rest % P;
    const int chain = (rest / P) * 8 + xcd;
    if (chain >= a.nchains) return;
    const int n = chain / a.H, h = chain % a.H;
    const int t0 = 0, t1 = a.T;
    const uint32_t ts = (uint32_t)a.H * D;
    const long long base = (long long)n * a.T * ts + (long long)h * D;
    const long long sbase = ((long long)n * a.H + h) * D * D;
    const uint4* crec = rec + (size_t)chain * nch * REC_PIECES;

    if (wave < NS) {
        const int vc = vblk * VB + wave * 16 + l16;
        uint32_t voff[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) voff[i] = ((uint32_t)(16 * (i >> 2) + 4 * grp + (i & 3)) * ts + vc) * 2u;
        uint32_t voff2[4];
        vpair_offsets(voff2, grp, vc, ts);
        f32x4 S[8];
        uint32_t vcur[8], vraw[4];
        auto vfetch = [&](uint32_t (&dst)[4], int cidx) {
            const int cs = t0 + cidx * C;
            const auto rv = chunk_rsrc(a.v, base + (long long)cs * ts, 2, min(C, t1 - cs), ts, D);
            vload(dst, rv, voff2);
        };
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                S[m][j] = a.h0 ? a.h0[sbase + (uint32_t)(16 * m + 4 * grp + j) * D + vc] : 0.f;
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __builtin_amdgcn_s_setprio(2);
        if (nch > 0) {
            vfetch(vraw, 0);
            vunpack(vcur, vraw, vc & 1);
        }
        __syncthreads();   // record 0 is in ops[0]
        for (int ci = 0; ci < nch; ++ci) {
            const int cs = t0 + ci * C;
            const int nv = min(C, t1 - cs);
            const Ops& op = ops[ci & 1].rec.op;
            if (ci + 1 < nch) vfetch(vraw, ci + 1);
            f32x4 Pt[2], Ot[2];
            state_products(S, op, ops[ci & 1].rec, l16, grp, Pt, Ot);
            const float4 bt0 = lds_vec<float4>(&op.beta[4 * grp]), bt1 = lds_vec<float4>(&op.beta[16 + 4 * grp]);
            const f16x4 ah = lds_vec<f16x4>(&op.A10[l16][tcol(l16, 8 * grp)]);   // A10 row l16, columns 4grp..4grp+3
            const auto ro = chunk_rsrc(a.o, base + (long long)cs * ts, 4, nv, ts, D);
            state_finish(S, op, Pt, Ot, vcur, bt0, bt1, ah, ro, voff, l16, grp);
            vunpack(vcur, vraw, vc & 1);
            __syncthreads();   // ops[ci & 1] is free, ops[(ci + 1) & 1] holds record ci+1
        }
        if (a.hT) {
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    a.hT[sbase + (uint32_t)(16 * m + 4 * grp + j) * D + vc] = S[m][j];
        }
    } else {
        // Two copy groups of NCW / 2 waves: group g moves the records of
        // parity g, so each group loads a record two chunks before it is due
        // and the load has two chunk periods to arrive. Lane i of a group
        // moves pieces i, i + CG_LANES, ... of a record.
        const int cg = (wave - NS) / (NCW / 2);
        const int cl = tid - 64 * NS - CG_LANES * cg;
        const u32x4* src = reinterpret_cast<const u32x4*>(crec) + cl;
        u32x4 r[CG_REGS];
        if (cg == 0) {
            if (nch > 0) {
                rec_load(r, src);
                rec_store(r, reinterpret_cast<u32x4*>(&ops[0]) + cl);
                if (nch > 2) rec_load(r, src + 2 * (size_t)REC_PIECES);
            }
        } else if (nch > 1) {
            rec_load(r, src + REC_PIECES);
        }
        __syncthreads();
        for (int ci = 0; ci < nch; ++ci) {
            const int rn = ci + 1;   // the record due in LDS by the end of this chunk
            if ((rn & 1) == cg && rn < nch) {
                rec_store(r, reinterpret_cast<u32x4*>(&ops[rn & 1]) + cl);
                if (rn + 2 < nch) rec_load(r, src + (size_t)(rn + 2) * REC_PIECES);
            }
            __syncthreads();
        }
    }
}



}  // namespace pipe

size_t two_pass_workspace(int nchains, int T) {
    const size_t nch = (size_t)((T + pipe::C - 1) / pipe::C);
    return (size_t)nchains * nch * sizeof(pipe::OpsBuf);
}

hipError_t launch_fwd_two_pass(const FwdArgs& a, void* workspace, int cus, hipStream_t stream) {
    const int nch = (a.T + pipe::C - 1) / pipe::C;
    if (a.nchains == 0) return hipSuccess;
    uint4* rec = static_cast<uint4*>(workspace);
    constexpr int per_wg = 16;
    if (nch > 0) {
        const int grid1 = a.nchains * ((nch + per_wg - 1) / per_wg);
        hipLaunchKernelGGL(pipe::kda_prep_pipe, dim3(grid1), dim3(64 * pipe::NH), 0, stream, a, rec, nch, per_wg);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int ns = min(4, pipe_state_waves(a.nchains, cus));   // the ablation keeps P >= 2
    const dim3 g3(pipe_workgroups(a.nchains, ns));
    if (ns == 1) hipLaunchKernelGGL((pipe::kda_recur_pipe<1>), g3, dim3(64 * (1 + pipe::NCW)), 0, stream, a, rec, nch);
    else if (ns == 2) hipLaunchKernelGGL((pipe::kda_recur_pipe<2>), g3, dim3(64 * (2 + pipe::NCW)), 0, stream, a, rec, nch);
    else hipLaunchKernelGGL((pipe::kda_recur_pipe<4>), g3, dim3(64 * (4 + pipe::NCW)), 0, stream, a, rec, nch);
    return hipGetLastError();
}

int pipe_state_waves(int nchains, int cus) {
    if ((long long)nchains * 8 <= cus) return 1;
    if ((long long)nchains * 4 <= cus) return 2;
    if ((long long)nchains * 2 <= cus) return 4;
    return 8;
}

int pipe_workgroups(int nchains, int state_waves) {
    const int groups = (nchains + 7) / 8;
    return groups * 8 * (D / (16 * state_waves));
}

hipError_t launch_fwd_pipe(const FwdArgs& a, int cus, hipStream_t stream) {
    const int ns = pipe_state_waves(a.nchains, cus);
    const int grid = pipe_workgroups(a.nchains, ns);
    if (grid == 0) return hipSuccess;
    const dim3 g3(grid);
    if (a.scalar_gate) {
        if (ns == 1) hipLaunchKernelGGL((pipe::kda_fwd_pipe<1, true>), g3, dim3(pipe::Split<1>::NT), 0, stream, a);
        else if (ns == 2) hipLaunchKernelGGL((pipe::kda_fwd_pipe<2, true>), g3, dim3(pipe::Split<2>::NT), 0, stream, a);
        else if (ns == 4) hipLaunchKernelGGL((pipe::kda_fwd_pipe<4, true>), g3, dim3(pipe::Split<4>::NT), 0, stream, a);
        else hipLaunchKernelGGL((pipe::kda_fwd_pipe<8, true>), g3, dim3(pipe::Split<8>::NT), 0, stream, a);
    } else {
        if (ns == 1) hipLaunchKernelGGL((pipe::kda_fwd_pipe<1, false>), g3, dim3(pipe::Split<1>::NT), 0, stream, a);
        else if (ns == 2) hipLaunchKernelGGL((pipe::kda_fwd_pipe<2, false>), g3, dim3(pipe::Split<2>::NT), 0, stream, a);
        else if (ns == 4) hipLaunchKernelGGL((pipe::kda_fwd_pipe<4, false>), g3, dim3(pipe::Split<4>::NT), 0, stream, a);
        else hipLaunchKernelGGL((pipe::kda_fwd_pipe<8, false>), g3, dim3(pipe::Split<8>::NT), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace kda
