// C-ABI entry points of libwoq: argument validation, workspace layout,
// descriptor staging and kernel sequencing on the caller's stream.
//
// Every argument check runs on the host before the first HIP call, so an
// invalid call enqueues nothing.  The first WOQ_WS_HEAD bytes of the
// caller's workspace are the status head (the non-finite weight count of the
// entropy and Sinkhorn calls).  Descriptor tables are built in host memory
// and copied in right after the head with one hipMemcpyAsync (pageable
// source: the runtime stages it before returning, so the host vector may go
// out of scope).  The rest of the workspace holds per-call scratch
// (histograms, reciprocal scales, Sinkhorn partials).
#include "launch.h"

#include <algorithm>
#include <cmath>
#include <mutex>
#include <tuple>
#include <cstring>
#include <vector>

using namespace woq;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;
constexpr int32_t kMaxMats = 1 << 20;
constexpr int32_t kMaxIters = 4096;
// Sinkhorn: matrices of one shape class run in one launch per iteration
// (MI355X's Infinity Cache serves re-reads barely faster than HBM, so there
// is no point in cache-sized groups; one big launch amortises everything).
constexpr int kSinqCUs = 256;          // MI355X compute units
// Widest Sinkhorn row: a workgroup pass holds 512 threads x 8 vectors of 8
// columns, with 1/t for the whole row in LDS.
constexpr int64_t kSinqMaxCols = 32768;
constexpr int kSinqWavesPerCU = 8;     // resident workgroup-pass waves per CU (2 per SIMD)

size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Workspace layouts start after the status head.
struct Arena {
    size_t off = WOQ_WS_HEAD;
    size_t take(size_t bytes, size_t a = kAlign) {
        off = align_up(off, a);
        const size_t o = off;
        off += bytes;
        return o;
    }
    size_t end() const { return align_up(off); }
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Row stride in elements (0 means contiguous).
int64_t eff_ld(const woq_mat& m) { return m.ld ? m.ld : m.cols; }

int32_t check_mats(const woq_mat* mats, int32_t n, bool cols8) {
    if (!mats) return WOQ_ERR_NULL;
    if (n < 1 || n > kMaxMats) return WOQ_ERR_COUNT;
    for (int32_t i = 0; i < n; ++i) {
        const woq_mat& m = mats[i];
        if (!m.data) return WOQ_ERR_NULL;
        if (m.dtype != WOQ_F32 && m.dtype != WOQ_BF16) return WOQ_ERR_DTYPE;
        if (m.reserved != 0 || m.rows < 1 || m.cols < 1 || m.ld < 0) return WOQ_ERR_SHAPE;
        const int64_t ld = eff_ld(m);
        // a strided matrix has 16-byte rows: ld and cols multiples of 8
        if (ld != m.cols && (ld < m.cols || ld % 8 || m.cols % 8)) return WOQ_ERR_SHAPE;
        if (m.rows > kMaxElems / ld) return WOQ_ERR_SHAPE;
        if (cols8 && (m.cols % 8)) return WOQ_ERR_SHAPE;
        if (!aligned(m.data, 16)) return WOQ_ERR_ALIGN;
    }
    return WOQ_OK;
}

// Copies the host-built descriptor tables [WOQ_WS_HEAD, end) into the
// workspace; the status head itself is not written.  On a stream that is
// being captured into a graph the bytes travel in kernel arguments (a
// captured copy from this pageable, short-lived buffer would be replayed
// after the buffer is gone); otherwise one asynchronous copy.
// zero_head: the copy starts at byte 0, so the status head is cleared by it
// (host[0, WOQ_WS_HEAD) holds zeros) instead of by a kernel of its own.
hipError_t stage_tables(void* ws, const std::vector<char>& host, size_t end, hipStream_t s,
                        bool zero_head = false) {
    const size_t from = zero_head ? 0 : WOQ_WS_HEAD;
    if (end <= from) return hipSuccess;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return e;
    if (cs != hipStreamCaptureStatusNone)
        return stage_bytes(static_cast<char*>(ws) + from, host.data() + from, end - from, s);
    return hipMemcpyAsync(static_cast<char*>(ws) + from, host.data() + from, end - from,
                          hipMemcpyHostToDevice, s);
}

// The call's non-finite weight counter (uint64 at byte 0 of the workspace).
unsigned long long* nonfinite_counter(void* ws) { return static_cast<unsigned long long*>(ws); }

int32_t check_ptrs(const void* const* arr, int32_t n, size_t align) {
    if (!arr) return WOQ_ERR_NULL;
    for (int32_t i = 0; i < n; ++i) {
        if (!arr[i]) return WOQ_ERR_NULL;
        if (!aligned(arr[i], align)) return WOQ_ERR_ALIGN;
    }
    return WOQ_OK;
}

int32_t check_opt_ptrs(const void* const* arr, int32_t n, size_t align) {
    if (!arr) return WOQ_OK;
    for (int32_t i = 0; i < n; ++i)
        if (arr[i] && !aligned(arr[i], align)) return WOQ_ERR_ALIGN;
    return WOQ_OK;
}

int32_t check_ws(const void* ws, size_t ws_bytes, size_t need) {
    if (!ws || !aligned(ws, kAlign) || ws_bytes < need) return WOQ_ERR_WORKSPACE;
    return WOQ_OK;
}

int64_t elems(const woq_mat& m) { return m.rows * m.cols; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <class T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }

// ------------------------------------------------------------------ entropy
struct EntLayout {
    int nb = 0, nf = 0;
    int slots = 0;          // bf16 histograms per batch
    int64_t units_b = 0, units_f = 0;
    size_t tab_b, ubeg_b, tab_f, ubeg_f, bmats, bbeg, nsz, table_end;
    size_t part_f, recs, lists, total;
};

// fp32: rows per entropy work unit of a strided matrix (0 for a contiguous
// one), and the matrix's number of work units.  bf16: the matrix's number
// of 16-byte vectors (the counting pass shares them out evenly).
int64_t ent_target(const woq_mat& m) {
    return std::min(kEntChunk, std::max(kEntMinChunk, cdiv(elems(m), kEntSplit)));
}
int32_t ent_rpu(const woq_mat& m) {
    return eff_ld(m) == m.cols ? 0 : (int32_t)std::max<int64_t>(1, ent_target(m) / m.cols);
}
int64_t ent_units(const woq_mat& m) {
    const int32_t rpu = ent_rpu(m);
    return rpu ? cdiv(m.rows, rpu) : cdiv(elems(m), ent_target(m));
}
// Elements per work unit of a contiguous matrix: the matrix split evenly
// (rounded up to a multiple of 8, so every unit starts 16-byte aligned).
int64_t ent_chunk(const woq_mat& m) {
    return ent_rpu(m) ? 0 : cdiv(cdiv(elems(m), ent_units(m)), 8) * 8;
}
int64_t ent_vectors(const woq_mat& m) {
    return eff_ld(m) == m.cols ? cdiv(elems(m), 8) : m.rows * (m.cols / 8);
}

// max_slots: at most this many bf16 matrices (a record and a list each,
// about 48 KiB) per batch.
EntLayout ent_layout(const woq_mat* mats, int32_t n, int32_t n_blocks, int max_slots = kHistSlots) {
    EntLayout L;
    for (int32_t i = 0; i < n; ++i) {
        if (mats[i].dtype == WOQ_BF16) { ++L.nb; L.units_b += ent_vectors(mats[i]); }
        else { ++L.nf; L.units_f += ent_units(mats[i]); }
    }
    Arena a;
    L.tab_b = a.take(sizeof(EntMat) * L.nb);
    L.ubeg_b = a.take(sizeof(int64_t) * (L.nb + 1));
    L.tab_f = a.take(sizeof(EntMat) * L.nf);
    L.ubeg_f = a.take(sizeof(int64_t) * (L.nf + 1));
    L.bmats = a.take(sizeof(int32_t) * n);
    L.bbeg = a.take(sizeof(int32_t) * (n_blocks + 1));
    L.nsz = a.take(sizeof(double) * n);
    L.table_end = a.end();
    L.part_f = a.take(sizeof(double) * 3 * L.units_f);
    L.slots = std::min(L.nb, max_slots);
    L.recs = a.take(sizeof(uint32_t) * kEntRecWords * (size_t)L.slots);
    L.lists = a.take(sizeof(uint16_t) * kEntListCap * (size_t)L.slots);
    L.total = a.end();
    return L;
}

// ------------------------------------------------------------------ sinkhorn
struct SinqGroup {
    int first = 0, count = 0, dtype = 0, cols_max = 0, max_strips = 0;
    SinqShape sh{0, 0, 0, 0};
    int64_t n_strips = 0, n_cunits = 0;
    size_t arr_off = 0;  // index of this group's first entry in sbeg / cbeg
};

struct SinqLayout {
    std::vector<int> order;          // table position -> caller's matrix index
    std::vector<int32_t> n_strips, strip_rows;  // per table position
    std::vector<SinqGroup> groups;
    size_t tab, sbeg, cbeg, table_end, total;
    std::vector<size_t> u, part;     // per table position
};

// shared: the call runs beside another on the same GPU (WOQ_SINQ_SHARED), so
// strips are planned for half of the resident workgroup slots.
SinqLayout sinq_layout(const woq_mat* mats, int32_t n, bool shared) {
    SinqLayout L;
    // launch sets: same dtype and same (threads, vectors per thread)
    std::vector<int> idx(n);
    for (int i = 0; i < n; ++i) idx[i] = i;
    auto key = [&](int i) {
        const SinqShape sh = sinq_shape((int)mats[i].cols, mats[i].dtype);
        return std::make_tuple(mats[i].dtype, sh.mode, sh.nv, sh.nt, sh.rag);
    };
    std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return key(a) < key(b); });
    L.order = idx;
    L.n_strips.assign(n, 0);
    L.strip_rows.assign(n, 0);
    int p = 0;
    while (p < n) {
        SinqGroup g;
        g.first = p;
        g.dtype = mats[idx[p]].dtype;
        g.sh = sinq_shape((int)mats[idx[p]].cols, mats[idx[p]].dtype);
        int q = p;
        while (q < n && key(idx[q]) == key(idx[p])) ++q;
        g.count = q - p;
        // Row strips per matrix.  Mode 0: a workgroup owns one strip of whole
        // register tiles (R rows).  Mode 1: it owns four strips' worth of
        // consecutive rows, dealt to its four waves in turn.  A workgroup
        // writes one partial row, so
        // n_strips counts workgroups.  Two plans, the faster estimate wins
        // (work counted in rows; cap = workgroups resident at once, about 8
        // waves per CU):
        //  A  one common strip height, the smallest for which every
        //     workgroup is resident at once (a single round);
        //  B  workgroups of about total / (rounds x cap) rows (at least 64),
        //     run in several rounds and scheduled as slots free up - better when
        //     the matrices are about as many as the slots, where plan A
        //     must give a whole large matrix to one workgroup.
        const int R = g.sh.mode == 1 ? 1 : sinq_tile_rows(g.dtype, g.sh.nv);
        const int per_wg = g.sh.mode == 1 ? 4 : 1;
        const int64_t unit = (int64_t)R * per_wg;  // rows per strip height step
        const int waves_per_wg = g.sh.mode == 1 ? 4 : g.sh.nt / 64;
        const int waves_per_cu =
            g.sh.mode == 1 ? 4 * sinq_wave_occupancy(g.dtype, g.sh.nv) : kSinqWavesPerCU;
        const int64_t full = (int64_t)kSinqCUs * std::max(1, waves_per_cu / waves_per_wg);
        const int64_t cap = shared ? std::max<int64_t>(1, full / 2) : full;
        int64_t total_rows = 0;
        for (int k = p; k < q; ++k) total_rows += mats[idx[k]].rows;
        // strip height (in tiles) of matrix k when its workgroups hold at
        // most t tiles per strip: an even split of the matrix
        auto height = [&](int64_t rows, int64_t t) {
            const int64_t n_wg = cdiv(rows, t * unit);
            return cdiv(cdiv(rows, n_wg), unit);
        };
        auto plan_cost = [&](int64_t t, int64_t* n_wg_out) {
            int64_t n_wg = 0, most = 0;
            for (int k = p; k < q; ++k) {
                const int64_t rows = mats[idx[k]].rows;
                const int64_t h = height(rows, t);
                n_wg += cdiv(rows, h * unit);
                most = std::max(most, h * unit);
            }
            *n_wg_out = n_wg;
            return n_wg <= cap ? most : cdiv(total_rows, cap) + most;
        };
        int64_t lo = 1, hi = 1;
        for (int k = p; k < q; ++k) hi = std::max<int64_t>(hi, cdiv(mats[idx[k]].rows, unit));
        while (lo < hi) {
            const int64_t mid = (lo + hi) / 2;
            int64_t n_wg = 0;
            plan_cost(mid, &n_wg);
            if (n_wg <= cap) hi = mid; else lo = mid + 1;
        }
        // plan B's rounds: 4 for the wave form (MoE stack: 3, 4, 6 rounds gave
        // 85.8, 84.0, 85.2 ms), 6 for the workgroup form (70B stack: 2, 4, 6,
        // 8 rounds gave 754, 712, 698-702, 702-703 ms)
        const int64_t rounds = g.sh.mode == 0 ? 6 : 4;
        const int64_t t_b = std::max<int64_t>(cdiv(64, unit), cdiv(total_rows, rounds * cap * unit));
        int64_t n_a = 0, n_b = 0;
        const int64_t cost_a = plan_cost(lo, &n_a), cost_b = plan_cost(t_b, &n_b);
        const int64_t t_sel = cost_b < cost_a ? t_b : lo;
        for (int k = p; k < q; ++k) {
            const woq_mat& m = mats[idx[k]];
            const int64_t srows = height(m.rows, t_sel) * R;
            L.strip_rows[k] = (int32_t)srows;
            L.n_strips[k] = (int32_t)cdiv(m.rows, srows * per_wg);
            g.n_strips += L.n_strips[k];
            g.max_strips = std::max<int>(g.max_strips, L.n_strips[k]);
            g.cols_max = std::max<int>(g.cols_max, (int)m.cols);
        }
        // A plan of several rounds (more workgroups than cap) ends in a
        // partial round.  The matrices dispatched in it (the last n_wg mod
        // cap workgroups, in table order) get strips of half the height, so
        // the last round runs half-size pieces (MoE stack: 85.7 -> 84.5 ms
        // per pass; 70B stack: 714-718 -> 702 ms; quarter-height strips, or
        // the last round and a half, measured the same or slower).
        if (g.n_strips > cap) {
            int64_t rem = g.n_strips % cap;
            for (int k = q - 1; k >= p && rem > 0; --k) {
                rem -= L.n_strips[k];
                const woq_mat& m = mats[idx[k]];
                const int64_t h = L.strip_rows[k] / R;   // register tiles per strip
                if (h < 2) continue;
                const int64_t srows = cdiv(h, 2) * R;
                const int32_t ns = (int32_t)cdiv(m.rows, srows * per_wg);
                g.n_strips += ns - L.n_strips[k];
                L.strip_rows[k] = (int32_t)srows;
                L.n_strips[k] = ns;
                g.max_strips = std::max<int>(g.max_strips, ns);
            }
        }
        const int rcols = 256 / sinq_reduce_slices(g.max_strips);
        // a wave-form matrix swept by one workgroup finishes its own columns
        for (int k = p; k < q; ++k)
            if (!(g.sh.mode == 1 && L.n_strips[k] == 1)) g.n_cunits += cdiv(mats[idx[k]].cols, rcols);
        L.groups.push_back(g);
        p = q;
    }
    Arena a;
    L.tab = a.take(sizeof(SinqMat) * n);
    const size_t narr = (size_t)n + L.groups.size();
    L.sbeg = a.take(sizeof(int64_t) * narr);
    L.cbeg = a.take(sizeof(int64_t) * narr);
    L.table_end = a.end();
    L.u.resize(n);
    L.part.resize(n);
    for (int k = 0; k < n; ++k) {
        const woq_mat& m = mats[idx[k]];
        const size_t psz = m.dtype == WOQ_BF16 ? sizeof(float2) : sizeof(float4);
        L.u[k] = a.take(sizeof(float) * m.cols, 64);
        L.part[k] = a.take(psz * (size_t)L.n_strips[k] * m.cols, 64);
    }
    size_t off = 0;
    for (auto& g : L.groups) { g.arr_off = off; off += g.count + 1; }
    L.total = a.end();
    return L;
}

// ------------------------------------------------------------------ quant
bool small_group(int32_t g) { return g >= 8 && g <= 512 && (g & (g - 1)) == 0; }

int32_t eff_group(const woq_mat& m, int32_t group) { return group ? group : (int32_t)m.cols; }

// group == 0 means one group per row.  quant additionally bounds large groups
// by what one workgroup keeps in registers.
int32_t check_group(const woq_mat* mats, int32_t n, int32_t group, bool quant) {
    if (group < 0 || (group && (group < 8 || group % 8))) return WOQ_ERR_SHAPE;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t g = eff_group(mats[i], group);
        if (mats[i].cols % g) return WOQ_ERR_SHAPE;
        if (quant && !(group && small_group(group))) {
            const int32_t lim = mats[i].dtype == WOQ_BF16 ? 32768 : 16384;
            if (g > lim) return WOQ_ERR_SHAPE;
        }
    }
    return WOQ_OK;
}

// Matrices are split into a bf16 list and an f32 list (one launch each).
struct QLayout {
    int nb = 0, nf = 0;
    size_t tab_b, ubeg_b, tab_f, ubeg_f, segs, ubeg_s, book, table_end, total;
    int64_t units_b = 0, units_f = 0, units_s = 0;
    int nseg = 0;
    int nsets = 0;               // quant: number of launch sets
    std::vector<size_t> rs, ct;  // per matrix, 0 = none
};

// Quantise launch sets: kernel kind 0 = row tiles (power-of-two groups of
// at most 512 columns), 1 = one wave per group (up to kQWaveMax columns,
// nvl 8-column vectors per lane), 2 = one workgroup per group.
struct QKey {
    int dtype, kind, nvl;
    bool operator<(const QKey& o) const {
        return std::tie(dtype, kind, nvl) < std::tie(o.dtype, o.kind, o.nvl);
    }
    bool operator==(const QKey& o) const { return dtype == o.dtype && kind == o.kind && nvl == o.nvl; }
};

QKey q_key(const woq_mat& m, int32_t group) {
    const int32_t g = eff_group(m, group);
    if (group && small_group(group)) return QKey{m.dtype, 0, 0};
    if (g <= kQWaveMax) {
        int nvl = 1;
        while (nvl * 64 * 8 < g) nvl *= 2;
        return QKey{m.dtype, 1, nvl};
    }
    return QKey{m.dtype, 2, 0};
}

int64_t q_units(const woq_mat& m, int32_t group) {
    const QKey k = q_key(m, group);
    const int64_t ng = elems(m) / eff_group(m, group);
    if (k.kind == 0) return cdiv(m.rows, kQTileRows) * cdiv(m.cols, kQTileCols);
    if (k.kind == 1) return cdiv(ng, 4);
    return ng;
}

// Ternary launch set: kind 1 = one wave per row (rows of at most
// kTernWaveMax columns, nvl 8-column vectors per lane), kind 2 = one
// workgroup per row.
QKey t_key(const woq_mat& m) {
    if (m.cols > kTernWaveMax) return QKey{m.dtype, 2, 0};
    int nvl = 1;
    while (nvl * 64 * 8 < m.cols) nvl *= 2;
    return QKey{m.dtype, 1, nvl};
}

int64_t t_units(const woq_mat& m) {
    return t_key(m).kind == 1 ? cdiv(m.rows, kTernRows) : m.rows;
}

// op: 0 quant, 1 dequant, 2 ternary.  For quant and ternary every matrix
// goes to the "b" table, ordered by launch set, and ubeg_b holds one offset
// run per set.
QLayout q_layout(const woq_mat* mats, int32_t n, int op, int32_t group,
                 const float* const* row_scale, const float* const* col_scale) {
    QLayout L;
    auto units = [&](const woq_mat& m) -> int64_t {
        if (op == 2) return t_units(m);
        if (op == 0) return q_units(m, group);
        return cdiv(m.rows, kDTileRows) * cdiv(m.cols, kQTileCols);
    };
    for (int32_t i = 0; i < n; ++i) {
        if (op != 1 || mats[i].dtype == WOQ_BF16) { ++L.nb; L.units_b += units(mats[i]); }
        else { ++L.nf; L.units_f += units(mats[i]); }
    }
    if (op != 1) {
        std::vector<QKey> keys;
        for (int32_t i = 0; i < n; ++i) keys.push_back(op == 0 ? q_key(mats[i], group) : t_key(mats[i]));
        std::sort(keys.begin(), keys.end());
        L.nsets = (int)(std::unique(keys.begin(), keys.end()) - keys.begin());
    }
    L.rs.assign(n, 0);
    L.ct.assign(n, 0);
    if (op == 0) {
        for (int32_t i = 0; i < n; ++i) {
            if (row_scale && row_scale[i]) { ++L.nseg; L.units_s += cdiv(mats[i].rows, 256); }
            if (col_scale && col_scale[i]) { ++L.nseg; L.units_s += cdiv(mats[i].cols, 256); }
        }
    }
    Arena a;
    L.tab_b = a.take(sizeof(QMat) * L.nb);
    L.ubeg_b = a.take(sizeof(int64_t) * (L.nb + std::max(L.nsets, 1)));
    L.tab_f = a.take(sizeof(QMat) * L.nf);
    L.ubeg_f = a.take(sizeof(int64_t) * (L.nf + 1));
    L.segs = a.take(sizeof(RecipSeg) * L.nseg);
    L.ubeg_s = a.take(sizeof(int64_t) * (L.nseg + 1));
    L.book = op < 2 ? a.take(sizeof(CbTable)) : 0;  // code-book grid (quant, dequant)
    L.table_end = a.end();
    if (op == 0) {
        for (int32_t i = 0; i < n; ++i) {
            if (row_scale && row_scale[i]) L.rs[i] = a.take(sizeof(float) * mats[i].rows, 64);
            if (col_scale && col_scale[i]) L.ct[i] = a.take(sizeof(float) * mats[i].cols, 64);
        }
    }
    L.total = a.end();
    return L;
}

// Code-book table from 2^bits levels (finite, strictly ascending): fp32
// midpoints, +inf padding, and per cell c of [-1, 1] (width 2 / kCbCells,
// left edge E_c = -1 + 2c / kCbCells) the count of midpoints certainly
// below y.  The kernel's cell index for y (mantissa bits of the fp32 sum
// y + 3, clamped to [2, 4)) is the true cell floor((y + 1) * kCbCells / 2)
// or a neighbour, and |y| <= 1 + 2^-23, so y lies in [E_{c-1}, E_{c+2}):
// midpoints below E_{c-1} are below y and midpoints at or above E_{c+2} are
// not.  Returns the comparisons per value (the widest spread), or -1 for an
// invalid book.
int cb_build(const float* levels, int bits, CbTable* t) {
    const int n = 1 << bits, nm = n - 1;
    for (int k = 0; k < n; ++k) {
        if (!std::isfinite(levels[k])) return -1;
        if (k && !(levels[k] > levels[k - 1])) return -1;
    }
    for (int k = 0; k < kCbMax; ++k) {
        t->level[k] = k < n ? levels[k] : 0.0f;
        t->mid[k] = k < nm ? (levels[k] + levels[k + 1]) * 0.5f : INFINITY;
    }
    auto below = [&](double e) {
        int c = 0;
        while (c < nm && (double)t->mid[c] < e) ++c;
        return c;
    };
    int steps = 1;
    for (int c = 0; c < kCbCells; ++c) {
        const double half = kCbCells / 2;
        const int lo = below(-1.0 + (c - 1) / half), hi = below(-1.0 + (c + 2) / half);
        t->lo[c] = (uint8_t)lo;
        steps = std::max(steps, hi - lo);
    }
    return steps;
}

// ------------------------------------------------------------------ DF11
struct DfSizes { int64_t n_seg, enc_bytes, gap_bytes, n_blocks; };
DfSizes df_sizes(int64_t total_bits) {
    DfSizes z;
    z.n_seg = cdiv(total_bits, 64);
    z.enc_bytes = 8 * z.n_seg + 8;
    z.gap_bytes = 4 * cdiv(5 * z.n_seg, 32) + 4;
    z.n_blocks = cdiv(z.n_seg, kDf11BlockSegs);
    return z;
}

// The lossless exponent code: contiguous BF16 matrices (the stream is in
// weight order, rows back to back).
int32_t check_bf16(const woq_mat* mats, int32_t n) {
    int32_t st = check_mats(mats, n, false);
    if (st) return st;
    for (int32_t i = 0; i < n; ++i) {
        if (mats[i].dtype != WOQ_BF16) return WOQ_ERR_DTYPE;
        if (eff_ld(mats[i]) != mats[i].cols) return WOQ_ERR_SHAPE;
    }
    return WOQ_OK;
}

// op: 0 histogram, 1 encode, 2 decode.  Table region (copied in one go):
// DfMat[n], DfCode[n] (encode), ubeg[n + 1], zbeg[n + 1] (encode); then the
// encode scratch (chunk totals and bases).
struct DfLayout {
    size_t tab, codes, ubeg, zbeg, table_end, bits, base, total;
    int64_t units = 0;
};
DfLayout df_layout(const woq_mat* mats, int32_t n, int op) {
    DfLayout L;
    Arena a;
    L.tab = a.take(sizeof(DfMat) * n);
    L.codes = op == 1 ? a.take(sizeof(DfCode) * n) : 0;
    L.ubeg = a.take(sizeof(int64_t) * (n + 1));
    L.zbeg = op == 1 ? a.take(sizeof(int64_t) * (n + 1)) : 0;
    L.table_end = a.end();
    for (int32_t i = 0; i < n; ++i) L.units += cdiv(elems(mats[i]), kDf11Chunk);
    L.bits = op == 1 ? a.take(sizeof(uint32_t) * L.units) : 0;
    L.base = op == 1 ? a.take(sizeof(int64_t) * L.units) : 0;
    L.total = a.end();
    return L;
}

// A codeword table must be a prefix code of lengths <= 32 with no code for
// the pointer exponents (Kraft sum <= 1, codewords within their lengths).
int32_t check_code(const uint8_t* len, const uint32_t* cw) {
    uint64_t kraft = 0;
    for (int s = 0; s < 256; ++s) {
        if (len[s] > kDf11MaxLen) return WOQ_ERR_VALUE;
        if (!len[s]) continue;
        if (s >= kDf11PtrMin) return WOQ_ERR_VALUE;
        if (len[s] < 32 && (cw[s] >> len[s])) return WOQ_ERR_VALUE;
        kraft += uint64_t(1) << (32 - len[s]);
    }
    return kraft <= (uint64_t(1) << 32) ? WOQ_OK : WOQ_ERR_VALUE;
}

#define WOQ_HIP(call)                                  \
    do {                                               \
        if ((call) != hipSuccess) return WOQ_ERR_HIP;  \
    } while (0)


// ------------------------------------------------------------ entropy calls
int32_t ent_check(const woq_mat* mats, int32_t n_mats, const int32_t* block_id, int32_t n_blocks,
                  const double* h_mat) {
    int32_t st = check_mats(mats, n_mats, false);
    if (st) return st;
    if (!h_mat) return WOQ_ERR_NULL;
    if (n_blocks < 1 || n_blocks > kMaxBlocks) return WOQ_ERR_COUNT;
    if (!block_id && n_blocks != 1) return WOQ_ERR_BLOCK;
    std::vector<int32_t> cnt(n_blocks, 0);
    for (int32_t i = 0; i < n_mats; ++i) {
        const int32_t b = block_id ? block_id[i] : 0;
        if (b < 0 || b >= n_blocks) return WOQ_ERR_BLOCK;
        ++cnt[b];
    }
    for (int32_t b = 0; b < n_blocks; ++b)
        if (!cnt[b]) return WOQ_ERR_BLOCK;
    return WOQ_OK;
}

// Enqueues the entropy computation with layout L in the scratch at ws
// (checked arguments).
int32_t ent_run(const EntLayout& L, const woq_mat* mats, int32_t n_mats, const int32_t* block_id,
                int32_t n_blocks, double x, double* h_mat, double* h_block, double* stats,
                int32_t* tier, int32_t* order, uint32_t* exp_hist, void* ws, hipStream_t stream) {
    std::vector<int32_t> cnt(n_blocks, 0);
    for (int32_t i = 0; i < n_mats; ++i) ++cnt[block_id ? block_id[i] : 0];
    std::vector<char> host(L.table_end, 0);
    EntMat* tb = at<EntMat>(host.data(), L.tab_b);
    EntMat* tf = at<EntMat>(host.data(), L.tab_f);
    int64_t* ub = at<int64_t>(host.data(), L.ubeg_b);
    int64_t* uf = at<int64_t>(host.data(), L.ubeg_f);
    int ib = 0, jf = 0;
    ub[0] = 0;
    uf[0] = 0;
    for (int32_t i = 0; i < n_mats; ++i) {
        const woq_mat& m = mats[i];
        EntMat e{m.data, elems(m), m.cols, eff_ld(m), m.dtype, i, (int32_t)m.rows, ent_rpu(m),
                 ent_chunk(m)};
        if (e.dtype == WOQ_BF16) { tb[ib] = e; ub[ib + 1] = ub[ib] + ent_vectors(m); ++ib; }
        else { tf[jf] = e; uf[jf + 1] = uf[jf] + ent_units(m); ++jf; }
    }
    int32_t* bm = at<int32_t>(host.data(), L.bmats);
    int32_t* bb = at<int32_t>(host.data(), L.bbeg);
    double* nsz = at<double>(host.data(), L.nsz);
    bb[0] = 0;
    for (int32_t b = 0; b < n_blocks; ++b) bb[b + 1] = bb[b] + cnt[b];
    std::vector<int32_t> fillp(bb, bb + n_blocks);
    for (int32_t i = 0; i < n_mats; ++i) {
        bm[fillp[block_id ? block_id[i] : 0]++] = i;
        nsz[i] = (double)elems(mats[i]);
    }

    WOQ_HIP(stage_tables(ws, host, L.table_end, stream, true));   // and the zeroed head
    unsigned long long* nf = nonfinite_counter(ws);
    const EntMat* dtb = at<EntMat>(ws, L.tab_b);
    const int64_t* dub = at<int64_t>(ws, L.ubeg_b);
    uint32_t* recs = at<uint32_t>(ws, L.recs);
    uint16_t* lists = at<uint16_t>(ws, L.lists);
    // batches of equal size, at most L.slots matrices each
    const int per = L.nb ? (int)cdiv(L.nb, cdiv(L.nb, L.slots)) : 0;
    for (int b0 = 0; b0 < L.nb; b0 += per) {
        const int b1 = std::min(L.nb, b0 + per);
        WOQ_HIP(fill_u32(recs, (size_t)(b1 - b0) * kEntRecWords, 0u, stream));
        WOQ_HIP(ent_hist_bf16(dtb + b0, dub + b0, b1 - b0, ub[b1] - ub[b0], recs, lists, stream));
        WOQ_HIP(ent_hist_final(dtb + b0, b1 - b0, recs, lists, h_mat, nf, exp_hist, stream));
    }
    if (L.nf)
        WOQ_HIP(ent_f32(at<EntMat>(ws, L.tab_f), at<int64_t>(ws, L.ubeg_f), L.nf, L.units_f,
                        at<double>(ws, L.part_f), h_mat, nf, exp_hist, stream));
    WOQ_HIP(ent_blocks(at<int32_t>(ws, L.bmats), at<int32_t>(ws, L.bbeg), at<double>(ws, L.nsz),
                       h_mat, n_blocks, x, h_block, stats, tier, order,
                       stream));
    return WOQ_OK;
}

// ------------------------------------------------------- static scratch
// Scratch of ewq_block_entropy_static, for callers that cannot allocate:
// one array per GPU the library runs on, held until the process ends.  In
// host code `scratch` names only a host-side stand-in; its device address
// is looked up once per device (with that device current) and kept in
// g_scratch, which is what kernels and copies receive.
constexpr size_t kStaticScratch = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratch];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

int32_t static_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WOQ_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WOQ_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return WOQ_OK;
}

}  // namespace

extern "C" {

const char* woq_status_string(int32_t s) {
    switch (s) {
        case WOQ_OK: return "ok";
        case WOQ_ERR_NULL: return "required pointer is NULL";
        case WOQ_ERR_SHAPE: return "shape / group / size constraint violated";
        case WOQ_ERR_DTYPE: return "unsupported dtype";
        case WOQ_ERR_BITS: return "bits must be 2, 3, 4 or 8";
        case WOQ_ERR_ITERS: return "iters out of range";
        case WOQ_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case WOQ_ERR_BLOCK: return "block id out of range or empty block";
        case WOQ_ERR_HIP: return "HIP call or kernel launch failed";
        case WOQ_ERR_ALIGN: return "pointer not sufficiently aligned";
        case WOQ_ERR_COUNT: return "matrix or block count out of range";
        case WOQ_ERR_VALUE: return "value not finite";
        case WOQ_ERR_SCRATCH: return "the call needs more than the library's static scratch array";
        default: return "unknown status";
    }
}

int32_t woq_workspace_size(int32_t op, const woq_mat* mats, int32_t n_mats, int32_t group,
                           size_t* bytes) {
    if (!bytes) return WOQ_ERR_NULL;
    int32_t st = check_mats(mats, n_mats, op != WOQ_OP_ENTROPY && op < WOQ_OP_DF11_HIST);
    if (st) return st;
    switch (op) {
        case WOQ_OP_ENTROPY: *bytes = ent_layout(mats, n_mats, kMaxBlocks).total; return WOQ_OK;
        case WOQ_OP_SINQ:
            for (int32_t i = 0; i < n_mats; ++i)
                if (mats[i].cols > kSinqMaxCols) return WOQ_ERR_SHAPE;
            // either plan (with or without WOQ_SINQ_SHARED)
            *bytes = std::max(sinq_layout(mats, n_mats, false).total,
                              sinq_layout(mats, n_mats, true).total);
            return WOQ_OK;
        case WOQ_OP_QUANT: {
            if ((st = check_group(mats, n_mats, group, true))) return st;
            // worst case: every matrix has both scale vectors
            std::vector<const float*> dummy(n_mats, reinterpret_cast<const float*>(16));
            *bytes = q_layout(mats, n_mats, 0, group, dummy.data(), dummy.data()).total;
            return WOQ_OK;
        }
        case WOQ_OP_DEQUANT:
            if ((st = check_group(mats, n_mats, group, false))) return st;
            *bytes = q_layout(mats, n_mats, 1, group, nullptr, nullptr).total;
            return WOQ_OK;
        case WOQ_OP_TERNARY: *bytes = q_layout(mats, n_mats, 2, 0, nullptr, nullptr).total; return WOQ_OK;
        case WOQ_OP_DF11_HIST: *bytes = df_layout(mats, n_mats, 0).total; return WOQ_OK;
        case WOQ_OP_DF11_ENCODE: *bytes = df_layout(mats, n_mats, 1).total; return WOQ_OK;
        case WOQ_OP_DF11_DECODE: *bytes = df_layout(mats, n_mats, 2).total; return WOQ_OK;
        default: return WOQ_ERR_SHAPE;
    }
}

int32_t ewq_block_entropy(const woq_mat* mats, int32_t n_mats, const int32_t* block_id,
                          int32_t n_blocks, double x, double* h_mat, double* h_block,
                          double* stats, int32_t* tier, int32_t* order, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
    int32_t st = ent_check(mats, n_mats, block_id, n_blocks, h_mat);
    if (st) return st;
    const EntLayout L = ent_layout(mats, n_mats, n_blocks);
    if ((st = check_ws(ws, ws_bytes, L.total))) return st;
    return ent_run(L, mats, n_mats, block_id, n_blocks, x, h_mat, h_block, stats, tier, order,
                   nullptr, ws, stream);
}

int32_t ewq_block_entropy_ex(const woq_mat* mats, int32_t n_mats, const int32_t* block_id,
                             int32_t n_blocks, double x, double* h_mat, double* h_block,
                             double* stats, int32_t* tier, int32_t* order, uint32_t* exp_hist,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
    int32_t st = ent_check(mats, n_mats, block_id, n_blocks, h_mat);
    if (st) return st;
    if (exp_hist && !aligned(exp_hist, 16)) return WOQ_ERR_ALIGN;
    const EntLayout L = ent_layout(mats, n_mats, n_blocks);
    if ((st = check_ws(ws, ws_bytes, L.total))) return st;
    return ent_run(L, mats, n_mats, block_id, n_blocks, x, h_mat, h_block, stats, tier, order,
                   exp_hist, ws, stream);
}

// The same computation with the library's static scratch array in place of
// a caller workspace (for callers that cannot allocate).  Histograms go
// through the array in batches of as many matrices as fit beside the tables.
int32_t ewq_block_entropy_static(const woq_mat* mats, int32_t n_mats, const int32_t* block_id,
                                 int32_t n_blocks, double x, double* h_mat, double* h_block,
                                 double* stats, int32_t* tier, int32_t* order,
                                 hipStream_t stream) {
    int32_t st = ent_check(mats, n_mats, block_id, n_blocks, h_mat);
    if (st) return st;
    EntLayout L = ent_layout(mats, n_mats, n_blocks, 0);   // tables and fp32 partials only
    if (L.total > kStaticScratch) return WOQ_ERR_SCRATCH;
    if (L.nb) {
        const size_t per_slot =
            sizeof(uint32_t) * kEntRecWords + sizeof(uint16_t) * kEntListCap + 2 * kAlign;
        const size_t fit = (kStaticScratch - L.total) / per_slot;
        if (fit < 1) return WOQ_ERR_SCRATCH;
        L = ent_layout(mats, n_mats, n_blocks, (int)std::min<size_t>(fit, kHistSlots));
        if (L.total > kStaticScratch) return WOQ_ERR_SCRATCH;
    }
    void* ws = nullptr;
    if ((st = static_scratch(&ws))) return st;
    return ent_run(L, mats, n_mats, block_id, n_blocks, x, h_mat, h_block, stats, tier, order,
                   nullptr, ws, stream);
}

int32_t sinq_balance(const woq_mat* mats, int32_t n_mats, int32_t iters, float* const* row_scale,
                     float* const* col_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
    return sinq_balance_ex(mats, n_mats, iters, 0, row_scale, col_scale, ws, ws_bytes, stream);
}

int32_t sinq_balance_ex(const woq_mat* mats, int32_t n_mats, int32_t iters, int32_t flags,
                        float* const* row_scale, float* const* col_scale, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
    int32_t st = check_mats(mats, n_mats, true);
    if (st) return st;
    for (int32_t i = 0; i < n_mats; ++i)
        if (mats[i].cols > kSinqMaxCols) return WOQ_ERR_SHAPE;
    if (iters < 0 || iters > kMaxIters) return WOQ_ERR_ITERS;
    if (flags & ~(WOQ_SINQ_RMS | WOQ_SINQ_SHARED)) return WOQ_ERR_VALUE;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(row_scale), n_mats, 4))) return st;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(col_scale), n_mats, 4))) return st;
    const SinqLayout L = sinq_layout(mats, n_mats, (flags & WOQ_SINQ_SHARED) != 0);
    if ((st = check_ws(ws, ws_bytes, L.total))) return st;

    unsigned long long* nf = nonfinite_counter(ws);
    if (iters == 0) {  // no weight is read
        WOQ_HIP(fill_u32(reinterpret_cast<uint32_t*>(nf), 2, 0u, stream));
        for (int32_t i = 0; i < n_mats; ++i) {
            WOQ_HIP(fill_f32(row_scale[i], (size_t)mats[i].rows, 1.0f, stream));
            WOQ_HIP(fill_f32(col_scale[i], (size_t)mats[i].cols, 1.0f, stream));
        }
        return WOQ_OK;
    }
    std::vector<char> host(L.table_end, 0);
    SinqMat* tab = at<SinqMat>(host.data(), L.tab);
    int64_t* sb = at<int64_t>(host.data(), L.sbeg);
    int64_t* cb = at<int64_t>(host.data(), L.cbeg);
    for (int32_t k = 0; k < n_mats; ++k) {
        const int i = L.order[k];
        const woq_mat& m = mats[i];
        SinqMat sm{};
        sm.data = m.data;
        sm.s = row_scale[i];
        sm.t = col_scale[i];
        sm.u = at<float>(ws, L.u[k]);
        sm.part = at<void>(ws, L.part[k]);
        sm.rows = (int32_t)m.rows;
        sm.cols = (int32_t)m.cols;
        sm.ld = (int32_t)eff_ld(m);
        sm.dtype = m.dtype;
        sm.n_strips = L.n_strips[k];
        sm.strip_rows = L.strip_rows[k];
        sm.rms = (flags & WOQ_SINQ_RMS) ? 1 : 0;
        tab[k] = sm;
    }
    for (const SinqGroup& g : L.groups) {
        int64_t* gs = sb + g.arr_off;
        int64_t* gc = cb + g.arr_off;
        gs[0] = gc[0] = 0;
        const int rcols = 256 / sinq_reduce_slices(g.max_strips);
        for (int k = 0; k < g.count; ++k) {
            const SinqMat& sm = tab[g.first + k];
            gs[k + 1] = gs[k] + sm.n_strips;
            gc[k + 1] = gc[k] + ((g.sh.mode == 1 && sm.n_strips == 1) ? 0 : cdiv(sm.cols, rcols));
        }
    }
    WOQ_HIP(stage_tables(ws, host, L.table_end, stream, true));   // and the zeroed head
    const SinqMat* dt = at<SinqMat>(ws, L.tab);
    const int64_t* dsb = at<int64_t>(ws, L.sbeg);
    const int64_t* dcb = at<int64_t>(ws, L.cbeg);
    for (const SinqGroup& g : L.groups)
        for (int32_t it = 0; it < iters; ++it)
            WOQ_HIP(sinq_iteration(dt + g.first, dsb + g.arr_off, dcb + g.arr_off, g.count,
                                   g.n_strips, g.n_cunits, g.max_strips, g.dtype, g.sh,
                                   g.cols_max, it == 0, nf, stream));
    return WOQ_OK;
}

}  // extern "C"

namespace {

// Quantisation on the affine grid (levels == NULL) or the code-book grid.
int32_t quant_impl(const woq_mat* mats, int32_t n_mats, const float* const* row_scale,
                   const float* const* col_scale, int32_t bits, int32_t group,
                   const float* levels, uint8_t* const* codes, float* const* scales,
                   uint8_t* const* zeros, void* ws, size_t ws_bytes, hipStream_t stream) {
    int32_t st = check_mats(mats, n_mats, true);
    if (st) return st;
    if (levels ? (bits < 2 || bits > 4) : (bits != 2 && bits != 3 && bits != 4 && bits != 8))
        return WOQ_ERR_BITS;
    if ((st = check_group(mats, n_mats, group, true))) return st;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(codes), n_mats, 16))) return st;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(scales), n_mats, 4))) return st;
    if (!levels && (st = check_ptrs(reinterpret_cast<const void* const*>(zeros), n_mats, 1))) return st;
    if ((st = check_opt_ptrs(reinterpret_cast<const void* const*>(row_scale), n_mats, 4))) return st;
    if ((st = check_opt_ptrs(reinterpret_cast<const void* const*>(col_scale), n_mats, 4))) return st;
    CbTable book;
    int steps = 0;
    if (levels && (steps = cb_build(levels, bits, &book)) < 0) return WOQ_ERR_VALUE;
    const QLayout L = q_layout(mats, n_mats, 0, group, row_scale, col_scale);
    if ((st = check_ws(ws, ws_bytes, L.total))) return st;

    std::vector<char> host(L.table_end, 0);
    if (levels) std::memcpy(host.data() + L.book, &book, sizeof(CbTable));
    const CbTable* dbook = levels ? at<CbTable>(ws, L.book) : nullptr;
    QMat* tb = at<QMat>(host.data(), L.tab_b);
    int64_t* ub = at<int64_t>(host.data(), L.ubeg_b);
    RecipSeg* sg = at<RecipSeg>(host.data(), L.segs);
    int64_t* us = at<int64_t>(host.data(), L.ubeg_s);
    us[0] = 0;
    int ks = 0;
    for (int32_t i = 0; i < n_mats; ++i) {
        const woq_mat& m = mats[i];
        if (L.rs[i]) {
            sg[ks] = RecipSeg{row_scale[i], at<float>(ws, L.rs[i]), m.rows, 0};
            us[ks + 1] = us[ks] + cdiv(m.rows, 256);
            ++ks;
        }
        if (L.ct[i]) {
            sg[ks] = RecipSeg{col_scale[i], at<float>(ws, L.ct[i]), m.cols, 0};
            us[ks + 1] = us[ks] + cdiv(m.cols, 256);
            ++ks;
        }
    }
    // matrices in launch-set order; each set has its own run of offsets
    std::vector<int> idx(n_mats);
    for (int32_t i = 0; i < n_mats; ++i) idx[i] = i;
    std::stable_sort(idx.begin(), idx.end(),
                     [&](int a, int b) { return q_key(mats[a], group) < q_key(mats[b], group); });
    struct Set { QKey key; int first, count; size_t uoff; int64_t units; bool tie; };
    std::vector<Set> sets;
    size_t uoff = 0;
    for (int p = 0; p < n_mats; ++p) {
        const int i = idx[p];
        const woq_mat& m = mats[i];
        const QKey key = q_key(m, group);
        if (sets.empty() || !(sets.back().key == key)) {
            if (!sets.empty()) uoff += sets.back().count + 1;
            sets.push_back(Set{key, p, 0, uoff, 0, bits == 8});
            ub[uoff] = 0;
        }
        Set& st_ = sets.back();
        QMat q{};
        q.data = m.data;
        q.codes = codes[i];
        q.scales = scales[i];
        q.zeros = levels ? nullptr : zeros[i];
        q.rs = L.rs[i] ? at<float>(ws, L.rs[i]) : nullptr;
        q.ct = L.ct[i] ? at<float>(ws, L.ct[i]) : nullptr;
        q.rows = (int32_t)m.rows;
        q.cols = (int32_t)m.cols;
        q.ld = (int32_t)eff_ld(m);
        q.dtype = m.dtype;
        q.group = eff_group(m, group);
        tb[p] = q;
        if (!q.rs && !q.ct) st_.tie = true;   // ratios of unscaled inputs can be exact halves
        ub[uoff + st_.count + 1] = ub[uoff + st_.count] + q_units(m, group);
        ++st_.count;
        st_.units = ub[uoff + st_.count];
    }
    // the code-book table, last in the tables, only when a book is used
    WOQ_HIP(stage_tables(ws, host, levels ? L.table_end : L.book, stream));
    if (L.nseg) WOQ_HIP(recip(at<RecipSeg>(ws, L.segs), at<int64_t>(ws, L.ubeg_s), L.nseg, us[L.nseg], stream));
    for (const Set& st_ : sets) {
        const QMat* dt = at<QMat>(ws, L.tab_b) + st_.first;
        const int64_t* du = at<int64_t>(ws, L.ubeg_b) + st_.uoff;
        if (st_.key.kind == 0)
            WOQ_HIP(quant_tile(dt, du, st_.count, st_.units, st_.key.dtype, bits, dbook, steps,
                               st_.tie, stream));
        else if (st_.key.kind == 1)
            WOQ_HIP(quant_wave(dt, du, st_.count, st_.units, st_.key.dtype, bits, st_.key.nvl, dbook,
                               steps, st_.tie, stream));
        else
            WOQ_HIP(quant_big(dt, du, st_.count, st_.units, st_.key.dtype, bits, dbook, steps,
                              st_.tie, stream));
    }
    return WOQ_OK;
}

// Dequantisation on the affine grid (levels == NULL) or the code-book grid.
int32_t dequant_impl(const woq_mat* out, int32_t n_mats, const uint8_t* const* codes,
                     const float* const* scales, const uint8_t* const* zeros,
                     const float* const* row_scale, const float* const* col_scale, int32_t bits,
                     int32_t group, const float* levels, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
    int32_t st = check_mats(out, n_mats, true);
    if (st) return st;
    if (levels ? (bits < 2 || bits > 4) : (bits != 2 && bits != 3 && bits != 4 && bits != 8))
        return WOQ_ERR_BITS;
    if ((st = check_group(out, n_mats, group, false))) return st;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(codes), n_mats, 16))) return st;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(scales), n_mats, 4))) return st;
    if ((st = check_opt_ptrs(reinterpret_cast<const void* const*>(row_scale), n_mats, 4))) return st;
    if ((st = check_opt_ptrs(reinterpret_cast<const void* const*>(col_scale), n_mats, 16))) return st;
    CbTable book;
    if (levels && cb_build(levels, bits, &book) < 0) return WOQ_ERR_VALUE;
    const QLayout L = q_layout(out, n_mats, 1, group, nullptr, nullptr);
    if ((st = check_ws(ws, ws_bytes, L.total))) return st;

    std::vector<char> host(L.table_end, 0);
    if (levels) std::memcpy(host.data() + L.book, &book, sizeof(CbTable));
    const CbTable* dbook = levels ? at<CbTable>(ws, L.book) : nullptr;
    QMat* tb = at<QMat>(host.data(), L.tab_b);
    QMat* tf = at<QMat>(host.data(), L.tab_f);
    int64_t* ub = at<int64_t>(host.data(), L.ubeg_b);
    int64_t* uf = at<int64_t>(host.data(), L.ubeg_f);
    ub[0] = uf[0] = 0;
    int ib = 0, jf = 0;
    for (int32_t i = 0; i < n_mats; ++i) {
        const woq_mat& m = out[i];
        QMat q{};
        q.data = m.data;
        q.codes = const_cast<uint8_t*>(codes[i]);
        q.scales = const_cast<float*>(scales[i]);
        q.zeros = zeros && !levels ? const_cast<uint8_t*>(zeros[i]) : nullptr;
        q.rs = row_scale ? row_scale[i] : nullptr;
        q.ct = col_scale ? col_scale[i] : nullptr;
        q.rows = (int32_t)m.rows;
        q.cols = (int32_t)m.cols;
        q.ld = (int32_t)eff_ld(m);
        q.dtype = m.dtype;
        q.group = eff_group(m, group);
        const int64_t u = cdiv(m.rows, kDTileRows) * cdiv(m.cols, kQTileCols);
        if (m.dtype == WOQ_BF16) { tb[ib] = q; ub[ib + 1] = ub[ib] + u; ++ib; }
        else { tf[jf] = q; uf[jf + 1] = uf[jf] + u; ++jf; }
    }
    // the code-book table, last in the tables, only when a book is used
    WOQ_HIP(stage_tables(ws, host, levels ? L.table_end : L.book, stream));
    if (L.nb) WOQ_HIP(dequant(at<QMat>(ws, L.tab_b), at<int64_t>(ws, L.ubeg_b), L.nb, ub[L.nb], WOQ_BF16, bits, dbook, stream));
    if (L.nf) WOQ_HIP(dequant(at<QMat>(ws, L.tab_f), at<int64_t>(ws, L.ubeg_f), L.nf, uf[L.nf], WOQ_F32, bits, dbook, stream));
    return WOQ_OK;
}

}  // namespace

extern "C" {

int32_t quant_pack_groupwise(const woq_mat* mats, int32_t n_mats, const float* const* row_scale,
                             const float* const* col_scale, int32_t bits, int32_t group,
                             uint8_t* const* codes, float* const* scales, uint8_t* const* zeros,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
    return quant_impl(mats, n_mats, row_scale, col_scale, bits, group, nullptr, codes, scales,
                      zeros, ws, ws_bytes, stream);
}

int32_t dequant_unpack(const woq_mat* out, int32_t n_mats, const uint8_t* const* codes,
                       const float* const* scales, const uint8_t* const* zeros,
                       const float* const* row_scale, const float* const* col_scale, int32_t bits,
                       int32_t group, void* ws, size_t ws_bytes, hipStream_t stream) {
    return dequant_impl(out, n_mats, codes, scales, zeros, row_scale, col_scale, bits, group,
                        nullptr, ws, ws_bytes, stream);
}

int32_t quant_pack_codebook(const woq_mat* mats, int32_t n_mats, const float* const* row_scale,
                            const float* const* col_scale, int32_t bits, int32_t group,
                            const float* levels, uint8_t* const* codes, float* const* scales,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!levels) return WOQ_ERR_NULL;
    return quant_impl(mats, n_mats, row_scale, col_scale, bits, group, levels, codes, scales,
                      nullptr, ws, ws_bytes, stream);
}

int32_t dequant_codebook(const woq_mat* out, int32_t n_mats, const uint8_t* const* codes,
                         const float* const* scales, const float* const* row_scale,
                         const float* const* col_scale, int32_t bits, int32_t group,
                         const float* levels, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!levels) return WOQ_ERR_NULL;
    return dequant_impl(out, n_mats, codes, scales, nullptr, row_scale, col_scale, bits, group,
                        levels, ws, ws_bytes, stream);
}

// Normal-quantile levels: l_k = P((k + 1/2) / n) / P((n - 1/2) / n), n =
// 2^bits, P the standard normal quantile, found by bisection on the normal
// CDF 0.5 erfc(-x / sqrt 2) in fp64 (to the last bit of the bracket), then
// rounded once to fp32.
int32_t woq_codebook_normal(int32_t bits, float* levels) {
    if (!levels) return WOQ_ERR_NULL;
    if (bits < 2 || bits > 4) return WOQ_ERR_BITS;
    const int n = 1 << bits;
    auto quantile = [](double p) {
        double lo = -40.0, hi = 40.0;
        for (int it = 0; it < 200; ++it) {
            const double mid = 0.5 * (lo + hi);
            if (mid <= lo || mid >= hi) break;
            if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p) lo = mid; else hi = mid;
        }
        return 0.5 * (lo + hi);
    };
    const double top = quantile((n - 0.5) / n);
    for (int k = 0; k < n; ++k) levels[k] = (float)(quantile((k + 0.5) / n) / top);
    return WOQ_OK;
}

int32_t ternary_pack(const woq_mat* mats, int32_t n_mats, uint8_t* const* codes,
                     float* const* row_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
    int32_t st = check_mats(mats, n_mats, true);
    if (st) return st;
    for (int32_t i = 0; i < n_mats; ++i)
        if (mats[i].cols > (mats[i].dtype == WOQ_BF16 ? 32768 : 16384)) return WOQ_ERR_SHAPE;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(codes), n_mats, 16))) return st;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(row_scale), n_mats, 4))) return st;
    const QLayout L = q_layout(mats, n_mats, 2, 0, nullptr, nullptr);
    if ((st = check_ws(ws, ws_bytes, L.total))) return st;

    std::vector<char> host(L.table_end, 0);
    QMat* tb = at<QMat>(host.data(), L.tab_b);
    int64_t* ub = at<int64_t>(host.data(), L.ubeg_b);
    // matrices in launch-set order; each set has its own run of offsets
    std::vector<int> idx(n_mats);
    for (int32_t i = 0; i < n_mats; ++i) idx[i] = i;
    std::stable_sort(idx.begin(), idx.end(),
                     [&](int a, int b) { return t_key(mats[a]) < t_key(mats[b]); });
    struct Set { QKey key; int first, count; size_t uoff; int64_t units; };
    std::vector<Set> sets;
    size_t uoff = 0;
    for (int p = 0; p < n_mats; ++p) {
        const int i = idx[p];
        const woq_mat& m = mats[i];
        const QKey key = t_key(m);
        if (sets.empty() || !(sets.back().key == key)) {
            if (!sets.empty()) uoff += sets.back().count + 1;
            sets.push_back(Set{key, p, 0, uoff, 0});
            ub[uoff] = 0;
        }
        Set& st_ = sets.back();
        QMat q{};
        q.data = m.data;
        q.codes = codes[i];
        q.scales = row_scale[i];
        q.rows = (int32_t)m.rows;
        q.cols = (int32_t)m.cols;
        q.ld = (int32_t)eff_ld(m);
        q.dtype = m.dtype;
        tb[p] = q;
        ub[uoff + st_.count + 1] = ub[uoff + st_.count] + t_units(m);
        ++st_.count;
        st_.units = ub[uoff + st_.count];
    }
    WOQ_HIP(stage_tables(ws, host, L.table_end, stream));
    for (const Set& st_ : sets) {
        const QMat* dt = at<QMat>(ws, L.tab_b) + st_.first;
        const int64_t* du = at<int64_t>(ws, L.ubeg_b) + st_.uoff;
        if (st_.key.kind == 1)
            WOQ_HIP(ternary_wave(dt, du, st_.count, st_.units, st_.key.dtype, st_.key.nvl, stream));
        else
            WOQ_HIP(ternary(dt, du, st_.count, st_.units, st_.key.dtype, stream));
    }
    return WOQ_OK;
}

int32_t ewq_budget_levels(const double* h_block, const int64_t* level_bytes, int32_t n_blocks,
                          int32_t n_levels, const int32_t* level0, int64_t budget,
                          int32_t* level_out, int64_t* total_out, int32_t* fits_out) {
    if (!h_block || !level_bytes || !level0 || !level_out || !total_out || !fits_out)
        return WOQ_ERR_NULL;
    if (n_blocks < 1 || n_blocks > (1 << 20) || n_levels < 1 || n_levels > 64) return WOQ_ERR_COUNT;
    if (budget < 0) return WOQ_ERR_SHAPE;
    for (int32_t b = 0; b < n_blocks; ++b) {
        if (level0[b] < 0 || level0[b] >= n_levels) return WOQ_ERR_SHAPE;
        for (int32_t l = 0; l < n_levels; ++l)
            if (level_bytes[(size_t)b * n_levels + l] < 0) return WOQ_ERR_SHAPE;
        if (!std::isfinite(h_block[b])) return WOQ_ERR_VALUE;
    }
    auto bytes = [&](int32_t b, int32_t l) { return level_bytes[(size_t)b * n_levels + l]; };
    std::vector<int32_t> lev(level0, level0 + n_blocks);
    int64_t total = 0;
    for (int32_t b = 0; b < n_blocks; ++b) total += bytes(b, lev[b]);
    std::vector<int32_t> by_h(n_blocks);
    for (int32_t b = 0; b < n_blocks; ++b) by_h[b] = b;
    if (total <= budget) {
        // promotion: scan blocks by descending entropy (ties: lower index);
        // the first one whose next level fits is raised, then scan again
        std::stable_sort(by_h.begin(), by_h.end(),
                         [&](int32_t a, int32_t c) { return h_block[a] > h_block[c]; });
        for (bool moved = true; moved;) {
            moved = false;
            for (int32_t b : by_h) {
                if (lev[b] + 1 >= n_levels) continue;
                const int64_t next = total - bytes(b, lev[b]) + bytes(b, lev[b] + 1);
                if (next <= budget) {
                    total = next;
                    ++lev[b];
                    moved = true;
                    break;
                }
            }
        }
    } else {
        // demotion: the lowest-entropy block above level 0 goes down a level
        std::stable_sort(by_h.begin(), by_h.end(),
                         [&](int32_t a, int32_t c) { return h_block[a] < h_block[c]; });
        size_t i = 0;
        while (total > budget && i < by_h.size()) {
            const int32_t b = by_h[i];
            if (lev[b] == 0) { ++i; continue; }
            total += bytes(b, lev[b] - 1) - bytes(b, lev[b]);
            --lev[b];
        }
    }
    std::copy(lev.begin(), lev.end(), level_out);
    *total_out = total;
    *fits_out = total <= budget ? 1 : 0;
    return WOQ_OK;
}

// ------------------------------------------------------------------ DF11
int32_t df11_buffer_sizes(int64_t n, int64_t total_bits, int64_t* n_seg, int64_t* enc_bytes,
                          int64_t* gap_bytes, int64_t* n_blocks) {
    if (!n_seg || !enc_bytes || !gap_bytes || !n_blocks) return WOQ_ERR_NULL;
    if (n < 1 || n > kMaxElems || total_bits < n || total_bits > kDf11MaxLen * n) return WOQ_ERR_SHAPE;
    const DfSizes z = df_sizes(total_bits);
    *n_seg = z.n_seg;
    *enc_bytes = z.enc_bytes;
    *gap_bytes = z.gap_bytes;
    *n_blocks = z.n_blocks;
    return WOQ_OK;
}

int32_t df11_build_code(const int64_t* hist, uint8_t* code_len, uint32_t* codeword,
                        uint8_t* tables, int32_t* n_tables, int64_t* total_bits) {
    if (!hist || !code_len || !codeword || !tables || !n_tables || !total_bits) return WOQ_ERR_NULL;
    int64_t sum = 0;
    for (int s = 0; s < 256; ++s) {
        if (hist[s] < 0 || hist[s] > kMaxElems) return WOQ_ERR_SHAPE;
        sum += hist[s];
    }
    if (sum > (int64_t(1) << 40)) return WOQ_ERR_SHAPE;
    return df11_code_build(hist, code_len, codeword, tables, n_tables, total_bits);
}

int32_t df11_exponent_histogram(const woq_mat* mats, int32_t n_mats, uint32_t* hist, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
    int32_t st = check_bf16(mats, n_mats);
    if (st) return st;
    if (!hist) return WOQ_ERR_NULL;
    if (!aligned(hist, 16)) return WOQ_ERR_ALIGN;
    const DfLayout L = df_layout(mats, n_mats, 0);
    if ((st = check_ws(ws, ws_bytes, L.total))) return st;
    std::vector<char> host(L.table_end, 0);
    DfMat* t = at<DfMat>(host.data(), L.tab);
    int64_t* ub = at<int64_t>(host.data(), L.ubeg);
    ub[0] = 0;
    for (int32_t i = 0; i < n_mats; ++i) {
        t[i].src = static_cast<const uint16_t*>(mats[i].data);
        t[i].n = elems(mats[i]);
        ub[i + 1] = ub[i] + cdiv(t[i].n, kDf11Chunk);
    }
    WOQ_HIP(stage_tables(ws, host, L.table_end, stream));
    WOQ_HIP(fill_u32(hist, (size_t)n_mats * 256, 0u, stream));
    WOQ_HIP(df11_hist(at<DfMat>(ws, L.tab), at<int64_t>(ws, L.ubeg), n_mats, ub[n_mats], hist, stream));
    return WOQ_OK;
}

int32_t df11_encode(const woq_mat* mats, int32_t n_mats, const uint8_t* const* code_len,
                    const uint32_t* const* codeword, const int64_t* total_bits,
                    uint8_t* const* enc, uint8_t* const* sign_mant, uint8_t* const* gaps,
                    uint32_t* const* block_pos, void* ws, size_t ws_bytes, hipStream_t stream) {
    int32_t st = check_bf16(mats, n_mats);
    if (st) return st;
    if (!code_len || !codeword || !total_bits) return WOQ_ERR_NULL;
    for (int32_t i = 0; i < n_mats; ++i) {
        if (!code_len[i] || !codeword[i]) return WOQ_ERR_NULL;
        if ((st = check_code(code_len[i], codeword[i]))) return st;
        const int64_t n = elems(mats[i]);
        if (total_bits[i] < n || total_bits[i] > kDf11MaxLen * n) return WOQ_ERR_SHAPE;
    }
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(enc), n_mats, 16))) return st;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(sign_mant), n_mats, 16))) return st;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(gaps), n_mats, 16))) return st;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(block_pos), n_mats, 4))) return st;
    const DfLayout L = df_layout(mats, n_mats, 1);
    if ((st = check_ws(ws, ws_bytes, L.total))) return st;

    std::vector<char> host(L.table_end, 0);
    DfMat* t = at<DfMat>(host.data(), L.tab);
    DfCode* c = at<DfCode>(host.data(), L.codes);
    int64_t* ub = at<int64_t>(host.data(), L.ubeg);
    int64_t* zb = at<int64_t>(host.data(), L.zbeg);
    ub[0] = zb[0] = 0;
    for (int32_t i = 0; i < n_mats; ++i) {
        const DfSizes z = df_sizes(total_bits[i]);
        DfMat& d = t[i];
        d.src = static_cast<const uint16_t*>(mats[i].data);
        d.enc = enc[i];
        d.sm = sign_mant[i];
        d.gaps = gaps[i];
        d.bpos = block_pos[i];
        d.n = elems(mats[i]);
        d.total_bits = total_bits[i];
        d.n_seg = z.n_seg;
        d.n_blocks = z.n_blocks;
        d.enc_bytes = z.enc_bytes;
        d.gap_bytes = z.gap_bytes;
        std::memcpy(c[i].code, codeword[i], sizeof(c[i].code));
        std::memcpy(c[i].len, code_len[i], sizeof(c[i].len));
        ub[i + 1] = ub[i] + cdiv(d.n, kDf11Chunk);
        zb[i + 1] = zb[i] + cdiv((z.enc_bytes + z.gap_bytes) / 4, 4096);
    }
    WOQ_HIP(stage_tables(ws, host, L.table_end, stream));
    WOQ_HIP(df11_encode_run(at<DfMat>(ws, L.tab), at<int64_t>(ws, L.ubeg), n_mats, ub[n_mats],
                            at<int64_t>(ws, L.zbeg), zb[n_mats], at<DfCode>(ws, L.codes),
                            at<uint32_t>(ws, L.bits), at<int64_t>(ws, L.base), stream));
    return WOQ_OK;
}

int32_t df11_decode(const woq_mat* out, int32_t n_mats, const uint8_t* const* enc,
                    const uint8_t* const* sign_mant, const uint8_t* const* gaps,
                    const uint32_t* const* block_pos, const uint8_t* const* tables,
                    const int32_t* n_tables, const uint8_t* const* code_len,
                    const int64_t* total_bits, void* ws, size_t ws_bytes, hipStream_t stream) {
    int32_t st = check_bf16(out, n_mats);
    if (st) return st;
    if (!n_tables || !total_bits) return WOQ_ERR_NULL;
    for (int32_t i = 0; i < n_mats; ++i) {
        if (n_tables[i] < 1 || n_tables[i] > kDf11MaxSub + 1) return WOQ_ERR_SHAPE;
        const int64_t n = elems(out[i]);
        if (total_bits[i] < n || total_bits[i] > kDf11MaxLen * n) return WOQ_ERR_SHAPE;
    }
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(enc), n_mats, 16))) return st;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(sign_mant), n_mats, 16))) return st;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(gaps), n_mats, 1))) return st;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(block_pos), n_mats, 4))) return st;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(tables), n_mats, 4))) return st;
    if ((st = check_ptrs(reinterpret_cast<const void* const*>(code_len), n_mats, 4))) return st;
    const DfLayout L = df_layout(out, n_mats, 2);
    if ((st = check_ws(ws, ws_bytes, L.total))) return st;

    std::vector<char> host(L.table_end, 0);
    DfMat* t = at<DfMat>(host.data(), L.tab);
    int64_t* ub = at<int64_t>(host.data(), L.ubeg);
    ub[0] = 0;
    for (int32_t i = 0; i < n_mats; ++i) {
        const DfSizes z = df_sizes(total_bits[i]);
        DfMat& d = t[i];
        d.dst = static_cast<uint16_t*>(out[i].data);
        d.enc = const_cast<uint8_t*>(enc[i]);
        d.sm = const_cast<uint8_t*>(sign_mant[i]);
        d.gaps = const_cast<uint8_t*>(gaps[i]);
        d.bpos = const_cast<uint32_t*>(block_pos[i]);
        d.tables = tables[i];
        d.lens = code_len[i];
        d.n = elems(out[i]);
        d.total_bits = total_bits[i];
        d.n_seg = z.n_seg;
        d.n_blocks = z.n_blocks;
        d.enc_bytes = z.enc_bytes;
        d.gap_bytes = z.gap_bytes;
        d.n_tables = n_tables[i];
        ub[i + 1] = ub[i] + z.n_blocks;
    }
    WOQ_HIP(stage_tables(ws, host, L.table_end, stream));
    WOQ_HIP(df11_decode_run(at<DfMat>(ws, L.tab), at<int64_t>(ws, L.ubeg), n_mats, ub[n_mats], stream));
    return WOQ_OK;
}

}  // extern "C"
