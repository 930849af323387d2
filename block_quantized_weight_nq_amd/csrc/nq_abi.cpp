// nq_abi.cpp -- the C ABI: closed format registry, the length rule, launch.
//
// Registry and rule: ONNX "DequantizePacked decoding specification",
// sections "Format identifiers" (27 case-sensitive identifiers, no
// parameters, unknown spellings are errors; the length rule) and
// "Quantization formats" (B, S); "nvfp4" is section 3.3 of the NInfer
// "tensor-formats" page carried as gguf:nvfp4 blocks plus a 4-byte binary32
// divisor.
#include <atomic>
#include <vector>
#include <string.h>

#include "../../include/nq.h"
#include "../../include/nq_measure.h"
#include "nq_fp8row.h"
#include "nq_gemv.h"
#include "nq_gqenc.h"
#include "nq_launch.h"

#define NQ_API extern "C" __attribute__((visibility("default")))

namespace {

struct Entry {
    const char *name;
    int family;
};

// Index = nq::Fmt id.
const Entry REGISTRY[nq::NUM_FORMATS] = {
    {"gguf:q4_0", NQ_FAMILY_SIMPLE},    {"gguf:q4_1", NQ_FAMILY_SIMPLE},
    {"gguf:q5_0", NQ_FAMILY_SIMPLE},    {"gguf:q5_1", NQ_FAMILY_SIMPLE},
    {"gguf:q8_0", NQ_FAMILY_SIMPLE},    {"gguf:q8_1", NQ_FAMILY_SIMPLE},
    {"gguf:q2_k", NQ_FAMILY_KQUANT},    {"gguf:q3_k", NQ_FAMILY_KQUANT},
    {"gguf:q4_k", NQ_FAMILY_KQUANT},    {"gguf:q5_k", NQ_FAMILY_KQUANT},
    {"gguf:q6_k", NQ_FAMILY_KQUANT},    {"gguf:q8_k", NQ_FAMILY_KQUANT},
    {"gguf:iq2_xxs", NQ_FAMILY_IQ},     {"gguf:iq2_xs", NQ_FAMILY_IQ},
    {"gguf:iq3_xxs", NQ_FAMILY_IQ},     {"gguf:iq1_s", NQ_FAMILY_IQ},
    {"gguf:iq4_nl", NQ_FAMILY_SIMPLE},  {"gguf:iq3_s", NQ_FAMILY_IQ},
    {"gguf:iq2_s", NQ_FAMILY_IQ},       {"gguf:iq4_xs", NQ_FAMILY_KQUANT},
    {"gguf:iq1_m", NQ_FAMILY_IQ},       {"gguf:tq1_0", NQ_FAMILY_TERNARY},
    {"gguf:tq2_0", NQ_FAMILY_TERNARY},  {"gguf:mxfp4", NQ_FAMILY_FP4},
    {"gguf:nvfp4", NQ_FAMILY_FP4},      {"gguf:q1_0", NQ_FAMILY_SIMPLE},
    {"gguf:q2_0", NQ_FAMILY_SIMPLE},    {"nvfp4", NQ_FAMILY_FP4},
};

constexpr int B_OF(int f) { return nq::block_values(f); }
constexpr int S_OF(int f) { return nq::block_bytes(f); }
constexpr int TRAILER_OF(int f) { return f == nq::NVFP4_DIV ? 4 : 0; }
constexpr uint64_t OUT_SIZE[4] = {4, 2, 2, 8};
constexpr uint64_t I64MAX = 0x7FFFFFFFFFFFFFFFull;

// a * b if it stays <= INT64_MAX.
bool mul_checked(uint64_t a, uint64_t b, uint64_t *r) {
    if (a != 0 && b > I64MAX / a) return false;
    *r = a * b;
    return true;
}

void fill_info(int id, nq_format_info *out) {
    out->id = id;
    out->name = REGISTRY[id].name;
    out->block_values = B_OF(id);
    out->block_bytes = S_OF(id);
    out->trailer_bytes = TRAILER_OF(id);
    out->family = REGISTRY[id].family;
}

// Compute units per device, looked up once per device.
constexpr int MAX_DEVICES = 64;
std::atomic<int> g_cu_count[MAX_DEVICES];

// Compute units of the current device.
uint32_t compute_units() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return 256;
    int cu = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cu <= 0) {
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
            cu = 256;
        g_cu_count[dev].store(cu, std::memory_order_relaxed);
    }
    return (uint32_t)cu;
}

// Workgroups the current device holds at once (the scale of the tile-size
// choice).
uint32_t resident_workgroups() { return compute_units() * NQ_RESIDENT_PER_CU; }

}  // namespace

NQ_API int nq_format_count(void) { return nq::NUM_FORMATS; }

NQ_API int nq_format_by_id(int32_t id, nq_format_info *out) {
    if (!out) return NQ_ERR_NULL_ARG;
    if (id < 0 || id >= nq::NUM_FORMATS) return NQ_ERR_UNKNOWN_FORMAT;
    fill_info(id, out);
    return NQ_OK;
}

NQ_API int nq_format_query(const char *name, nq_format_info *out) {
    if (!name || !out) return NQ_ERR_NULL_ARG;
    for (int id = 0; id < nq::NUM_FORMATS; id++) {
        if (strcmp(REGISTRY[id].name, name) == 0) {
            fill_info(id, out);
            return NQ_OK;
        }
    }
    return NQ_ERR_UNKNOWN_FORMAT;
}

NQ_API int nq_validate(int32_t format, uint64_t nbytes, const int64_t *shape, int32_t rank,
                       int32_t out_dtype, uint64_t *out_elems, uint64_t *out_bytes) {
    if (format < 0 || format >= nq::NUM_FORMATS) return NQ_ERR_UNKNOWN_FORMAT;
    if (out_dtype < NQ_F32 || out_dtype > NQ_F64) return NQ_ERR_BAD_DTYPE;
    if (rank < 1) return NQ_ERR_BAD_RANK;
    if (!shape) return NQ_ERR_NULL_ARG;
    bool empty = false;
    for (int32_t i = 0; i < rank; i++) {
        if (shape[i] < 0) return NQ_ERR_BAD_DIM;
        if (shape[i] == 0) empty = true;
    }
    const uint64_t B = (uint64_t)B_OF(format), S = (uint64_t)S_OF(format);
    const uint64_t K = (uint64_t)shape[rank - 1];
    if (K % B != 0) return NQ_ERR_NOT_BLOCK_ALIGNED;
    uint64_t elems = 0, bytes = 0;
    if (!empty) {
        uint64_t rows = 1, blocks = 0, wide = 0;
        for (int32_t i = 0; i + 1 < rank; i++)
            if (!mul_checked(rows, (uint64_t)shape[i], &rows)) return NQ_ERR_OVERFLOW;
        if (!mul_checked(rows, K / B, &blocks) || !mul_checked(blocks, S, &bytes) ||
            !mul_checked(rows, K, &elems) || !mul_checked(elems, 8, &wide))
            return NQ_ERR_OVERFLOW;
    }
    bytes += (uint64_t)TRAILER_OF(format);
    if (bytes > I64MAX) return NQ_ERR_OVERFLOW;
    if (nbytes != bytes) return NQ_ERR_LENGTH_MISMATCH;
    if (out_elems) *out_elems = elems;
    if (out_bytes) *out_bytes = elems * OUT_SIZE[out_dtype];
    return NQ_OK;
}

namespace {

// Pointer checks and the launch, after validation.  ndiv divisor words
// close an "nvfp4" payload; each covers gu units (rows per source * K / 8).
int launch_validated(int32_t format, const void *payload, uint64_t nbytes, uint64_t elems, int32_t out_dtype,
                     void *out, uint32_t ndiv, uint64_t gu, hipStream_t stream) {
    if (nbytes > 0 && !payload) return NQ_ERR_NULL_ARG;
    if (elems == 0) return NQ_OK;
    if (!out) return NQ_ERR_NULL_ARG;
    if (((uintptr_t)out % OUT_SIZE[out_dtype]) != 0) return NQ_ERR_MISALIGNED;
    nq::LaunchArgs L;
    L.payload = (const uint8_t *)payload;
    L.nbytes = nbytes;
    L.nblocks = elems / (uint64_t)B_OF(format);
    L.out = out;
    L.resident = resident_workgroups();
    L.ndiv = ndiv;
    L.gu = gu;
    switch (REGISTRY[format].family) {
    case NQ_FAMILY_SIMPLE: return nq::launch_simple(format, out_dtype, L, stream);
    case NQ_FAMILY_KQUANT: return nq::launch_kquant(format, out_dtype, L, stream);
    case NQ_FAMILY_IQ: return nq::launch_iq(format, out_dtype, L, stream);
    case NQ_FAMILY_FP4: return nq::launch_fp4(format, out_dtype, L, stream);
    default: return nq::launch_ternary(format, out_dtype, L, stream);
    }
}

constexpr int64_t MAX_DIVISORS = (int64_t)1 << 30;

}  // namespace

NQ_API int nq_dequantize_packed(int32_t format, const void *payload, uint64_t nbytes, const int64_t *shape,
                                int32_t rank, int32_t out_dtype, void *out, hipStream_t stream) {
    uint64_t elems = 0;
    const int st = nq_validate(format, nbytes, shape, rank, out_dtype, &elems, nullptr);
    if (st != NQ_OK) return st;
    // one divisor: its group is the whole tensor
    return launch_validated(format, payload, nbytes, elems, out_dtype, out, 1u, elems / 8 ? elems / 8 : 1, stream);
}

namespace {

int launch_many_family(int32_t format, int ot, bool vec, const nq::ManyItem *items, int n, hipStream_t stream) {
    const uint32_t resident = resident_workgroups();
    switch (REGISTRY[format].family) {
    case NQ_FAMILY_SIMPLE: return nq::launch_many_simple(format, ot, vec, items, n, resident, stream);
    case NQ_FAMILY_KQUANT: return nq::launch_many_kquant(format, ot, vec, items, n, resident, stream);
    case NQ_FAMILY_IQ: return nq::launch_many_iq(format, ot, vec, items, n, resident, stream);
    case NQ_FAMILY_FP4: return nq::launch_many_fp4(format, ot, vec, items, n, resident, stream);
    default: return nq::launch_many_ternary(format, ot, vec, items, n, resident, stream);
    }
}

}  // namespace

NQ_API int nq_dequantize_packed_many(const nq_tensor *tensors, int32_t count, int32_t out_dtype, int32_t *failed,
                                     hipStream_t stream) {
    if (failed) *failed = -1;
    if (count < 0) return NQ_ERR_BAD_DIM;
    if (count > 0 && !tensors) return NQ_ERR_NULL_ARG;
    if (out_dtype < NQ_F32 || out_dtype > NQ_F64) return NQ_ERR_BAD_DTYPE;
    // every tensor is checked before anything is launched
    std::vector<uint64_t> elems((size_t)count);
    for (int32_t i = 0; i < count; i++) {
        const nq_tensor &t = tensors[i];
        int st = nq_validate(t.format, t.nbytes, t.shape, t.rank, out_dtype, &elems[(size_t)i], nullptr);
        if (st == NQ_OK && t.nbytes > 0 && !t.payload) st = NQ_ERR_NULL_ARG;
        if (st == NQ_OK && elems[(size_t)i] > 0 && !t.out) st = NQ_ERR_NULL_ARG;
        if (st == NQ_OK && elems[(size_t)i] > 0 && (uintptr_t)t.out % OUT_SIZE[out_dtype] != 0)
            st = NQ_ERR_MISALIGNED;
        if (st != NQ_OK) {
            if (failed) *failed = i;
            return st;
        }
    }
    // one group per (format, 16-byte aligned output or not), in order of first appearance
    std::vector<char> done((size_t)count, 0);
    std::vector<nq::ManyItem> group;
    for (int32_t i = 0; i < count; i++) {
        if (done[(size_t)i] || elems[(size_t)i] == 0) continue;
        const int32_t f = tensors[i].format;
        const bool vec = ((uintptr_t)tensors[i].out & 15u) == 0;
        group.clear();
        for (int32_t j = i; j < count; j++) {
            const nq_tensor &t = tensors[j];
            if (done[(size_t)j] || elems[(size_t)j] == 0 || t.format != f || (((uintptr_t)t.out & 15u) == 0) != vec)
                continue;
            done[(size_t)j] = 1;
            nq::ManyItem it;
            it.payload = (const uint8_t *)t.payload;
            it.nbytes = t.nbytes;
            it.nblocks = elems[(size_t)j] / (uint64_t)B_OF(f);
            it.out = t.out;
            group.push_back(it);
        }
        const int st = launch_many_family(f, out_dtype, vec, group.data(), (int)group.size(), stream);
        if (st != NQ_OK) return st;
    }
    return NQ_OK;
}

NQ_API int nq_measure_stream(const void *src, uint64_t src_bytes, void *dst, uint64_t dst_bytes,
                             int32_t chunks_per_thread, int32_t flags, hipStream_t stream) {
    if (!src || !dst) return NQ_ERR_NULL_ARG;
    if ((uintptr_t)src % 16 != 0 || (uintptr_t)dst % 16 != 0) return NQ_ERR_MISALIGNED;
    if (dst_bytes == 0 || src_bytes > dst_bytes || src_bytes % 16 != 0 || dst_bytes % 16 != 0)
        return NQ_ERR_BAD_DIM;
    const int c = chunks_per_thread;
    if ((c != 1 && c != 2 && c != 4 && c != 8) || (flags & ~3) != 0) return NQ_ERR_BAD_DIM;
    if (dst_bytes > (1ull << 40)) return NQ_ERR_OVERFLOW;
    return nq::launch_stream(src, src_bytes, dst, dst_bytes, c, (flags & NQ_STREAM_NT_LOAD) != 0,
                             (flags & NQ_STREAM_NT_STORE) != 0, stream);
}

NQ_API int nq_validate_nvfp4_stacked(uint64_t nbytes, const int64_t *shape, int32_t rank, int64_t divisors,
                                     int32_t out_dtype, uint64_t *out_elems, uint64_t *out_bytes) {
    if (out_dtype < NQ_F32 || out_dtype > NQ_F64) return NQ_ERR_BAD_DTYPE;
    if (rank < 1) return NQ_ERR_BAD_RANK;
    if (!shape) return NQ_ERR_NULL_ARG;
    for (int32_t i = 0; i < rank; i++)
        if (shape[i] < 0) return NQ_ERR_BAD_DIM;
    if (shape[rank - 1] % 64 != 0) return NQ_ERR_NOT_BLOCK_ALIGNED;
    if (divisors < 1 || divisors > MAX_DIVISORS) return NQ_ERR_BAD_DIVISORS;
    // the single-divisor rule fixes every count except the trailer
    uint64_t elems = 0, bytes1 = 0, rows = 1;
    const int st = nq_validate(nq::NVFP4_DIV, 0, shape, rank, out_dtype, nullptr, nullptr);
    if (st != NQ_OK && st != NQ_ERR_LENGTH_MISMATCH) return st;
    for (int32_t i = 0; i + 1 < rank; i++)
        if (!mul_checked(rows, (uint64_t)shape[i], &rows)) return NQ_ERR_OVERFLOW;
    if (rows % (uint64_t)divisors != 0) return NQ_ERR_BAD_DIVISORS;
    for (int32_t i = 0; i < rank; i++)
        if (shape[i] == 0) rows = 0;
    if (rows != 0) {
        const uint64_t K = (uint64_t)shape[rank - 1];
        elems = rows * K;                 // bounded by nq_validate
        bytes1 = rows * (K / 64) * 36;
    }
    const uint64_t bytes = bytes1 + 4 * (uint64_t)divisors;
    if (bytes > I64MAX) return NQ_ERR_OVERFLOW;
    if (nbytes != bytes) return NQ_ERR_LENGTH_MISMATCH;
    if (out_elems) *out_elems = elems;
    if (out_bytes) *out_bytes = elems * OUT_SIZE[out_dtype];
    return NQ_OK;
}

NQ_API int nq_dequantize_nvfp4_stacked(const void *payload, uint64_t nbytes, const int64_t *shape, int32_t rank,
                                       int64_t divisors, int32_t out_dtype, void *out, hipStream_t stream) {
    uint64_t elems = 0;
    const int st = nq_validate_nvfp4_stacked(nbytes, shape, rank, divisors, out_dtype, &elems, nullptr);
    if (st != NQ_OK) return st;
    const uint64_t gu = elems / 8 / (uint64_t)divisors;  // units per source; 0 only when empty
    return launch_validated(nq::NVFP4_DIV, payload, nbytes, elems, out_dtype, out, (uint32_t)divisors,
                            gu ? gu : 1, stream);
}

NQ_API int nq_validate_fp8_row(int32_t scale_kind, uint64_t nbytes, const int64_t *shape, int32_t rank,
                               int32_t out_dtype, uint64_t *out_elems, uint64_t *out_bytes) {
    if (scale_kind != NQ_FP8_ROW_BF16 && scale_kind != NQ_FP8_ROW_FP16) return NQ_ERR_UNKNOWN_FORMAT;
    if (out_dtype < NQ_F32 || out_dtype > NQ_F64) return NQ_ERR_BAD_DTYPE;
    if (rank != 2) return NQ_ERR_BAD_RANK;
    if (!shape) return NQ_ERR_NULL_ARG;
    if (shape[0] <= 0 || shape[1] <= 0) return NQ_ERR_BAD_DIM;
    uint64_t elems = 0, wide = 0, scale_bytes = 0;
    if (!mul_checked((uint64_t)shape[0], (uint64_t)shape[1], &elems) || !mul_checked(elems, 8, &wide) ||
        !mul_checked((uint64_t)shape[0], 2, &scale_bytes) || elems > I64MAX - scale_bytes)
        return NQ_ERR_OVERFLOW;
    if (nbytes != elems + scale_bytes) return NQ_ERR_LENGTH_MISMATCH;
    if (out_elems) *out_elems = elems;
    if (out_bytes) *out_bytes = elems * OUT_SIZE[out_dtype];
    return NQ_OK;
}

NQ_API int nq_dequantize_fp8_row(int32_t scale_kind, const void *payload, uint64_t nbytes, const int64_t *shape,
                                 int32_t rank, int32_t out_dtype, void *out, hipStream_t stream) {
    uint64_t elems = 0;
    const int st = nq_validate_fp8_row(scale_kind, nbytes, shape, rank, out_dtype, &elems, nullptr);
    if (st != NQ_OK) return st;
    if (!payload || !out) return NQ_ERR_NULL_ARG;  // both dimensions are positive: never empty
    if (((uintptr_t)out % OUT_SIZE[out_dtype]) != 0) return NQ_ERR_MISALIGNED;
    nq::F8Launch L;
    L.payload = (const uint8_t *)payload;
    L.N = (uint64_t)shape[0];
    L.K = (uint64_t)shape[1];
    L.out = out;
    return nq::launch_fp8_row(scale_kind, out_dtype, L, stream);
}

NQ_API int nq_validate_grouped_absmax(int32_t scheme, const int64_t *shape, int32_t rank, int32_t in_dtype,
                                      uint64_t *codes_bytes, uint64_t *scales_bytes) {
    if (scheme < NQ_GQ_Q4_G64 || scheme > NQ_GQ_Q8_G32) return NQ_ERR_UNKNOWN_FORMAT;
    if (in_dtype < NQ_F32 || in_dtype > NQ_F64) return NQ_ERR_BAD_DTYPE;
    if (rank != 2) return NQ_ERR_BAD_RANK;
    if (!shape) return NQ_ERR_NULL_ARG;
    if (shape[0] <= 0 || shape[1] <= 0) return NQ_ERR_BAD_DIM;
    const uint64_t N = (uint64_t)shape[0], K = (uint64_t)shape[1], G = (uint64_t)nq::GQ[scheme].G;
    uint64_t elems = 0, in_bytes = 0, ngroups = 0, sbytes = 0;
    if (K >= (1ull << 31) || !mul_checked(N, K, &elems) || !mul_checked(elems, OUT_SIZE[in_dtype], &in_bytes) ||
        !mul_checked(N, (K + G - 1) / G, &ngroups) || !mul_checked(ngroups, 2, &sbytes))
        return NQ_ERR_OVERFLOW;
    if (codes_bytes) *codes_bytes = elems;
    if (scales_bytes) *scales_bytes = sbytes;
    return NQ_OK;
}

NQ_API int nq_quantize_grouped_absmax(int32_t scheme, const void *x, const int64_t *shape, int32_t rank,
                                      int32_t in_dtype, void *codes, void *scales, uint32_t *status,
                                      hipStream_t stream) {
    const int st = nq_validate_grouped_absmax(scheme, shape, rank, in_dtype, nullptr, nullptr);
    if (st != NQ_OK) return st;
    if (!x || !codes || !scales || !status) return NQ_ERR_NULL_ARG;
    if ((uintptr_t)x % OUT_SIZE[in_dtype] != 0 || (uintptr_t)scales % 2 != 0 || (uintptr_t)status % 4 != 0)
        return NQ_ERR_MISALIGNED;
    nq::GqLaunch L;
    L.x = x;
    L.codes = (int8_t *)codes;
    L.scales = (uint16_t *)scales;
    L.status = status;
    L.N = (uint64_t)shape[0];
    L.K = (uint64_t)shape[1];
    return nq::launch_grouped_absmax(scheme, in_dtype, L, stream);
}

NQ_API int nq_validate_quantize_q8_1(const int64_t *shape, int32_t rank, int32_t in_dtype,
                                     uint64_t *blocks_bytes) {
    if (in_dtype < NQ_F32 || in_dtype > NQ_F64) return NQ_ERR_BAD_DTYPE;
    if (rank != 2) return NQ_ERR_BAD_RANK;
    if (!shape) return NQ_ERR_NULL_ARG;
    if (shape[0] <= 0 || shape[1] <= 0) return NQ_ERR_BAD_DIM;
    if (shape[1] % 32 != 0) return NQ_ERR_NOT_BLOCK_ALIGNED;
    uint64_t elems = 0, in_bytes = 0, blocks = 0, bytes = 0;
    if (!mul_checked((uint64_t)shape[0], (uint64_t)shape[1], &elems) ||
        !mul_checked(elems, OUT_SIZE[in_dtype], &in_bytes) ||
        !mul_checked((uint64_t)shape[0], (uint64_t)shape[1] / 32, &blocks) || !mul_checked(blocks, 36, &bytes))
        return NQ_ERR_OVERFLOW;
    if (blocks_bytes) *blocks_bytes = bytes;
    return NQ_OK;
}

NQ_API int nq_quantize_q8_1(const void *x, const int64_t *shape, int32_t rank, int32_t in_dtype, void *blocks,
                            uint32_t *status, hipStream_t stream) {
    const int st = nq_validate_quantize_q8_1(shape, rank, in_dtype, nullptr);
    if (st != NQ_OK) return st;
    if (!x || !blocks || !status) return NQ_ERR_NULL_ARG;
    if ((uintptr_t)x % OUT_SIZE[in_dtype] != 0 || (uintptr_t)blocks % 4 != 0 || (uintptr_t)status % 4 != 0)
        return NQ_ERR_MISALIGNED;
    nq::Q81Launch L;
    L.x = x;
    L.nblocks = (uint64_t)shape[0] * ((uint64_t)shape[1] / 32);
    L.blocks = (uint32_t *)blocks;
    L.status = status;
    return nq::launch_quantize_q8_1(in_dtype, L, stream);
}

static int launch_gemv_family(int32_t format, const nq::GvLaunch &L, hipStream_t stream) {
    switch (REGISTRY[format].family) {
    case NQ_FAMILY_SIMPLE: return nq::launch_gemv_simple(format, L, stream);
    case NQ_FAMILY_KQUANT: return nq::launch_gemv_kquant(format, L, stream);
    case NQ_FAMILY_IQ: return nq::launch_gemv_iq(format, L, stream);
    default: return nq::launch_gemv_fp4t(format, L, stream);
    }
}

NQ_API int nq_validate_gemv_q8_1(int32_t format, uint64_t nbytes, int64_t N, int64_t K, int64_t M) {
    if (format < 0 || format >= nq::NUM_FORMATS || TRAILER_OF(format) != 0) return NQ_ERR_UNKNOWN_FORMAT;
    if (N <= 0 || K <= 0 || M <= 0 || M > nq::GV_MAX_M) return NQ_ERR_BAD_DIM;
    if (K % B_OF(format) != 0) return NQ_ERR_NOT_BLOCK_ALIGNED;
    if (N >= (1ll << 31) || K >= (1ll << 31)) return NQ_ERR_OVERFLOW;
    uint64_t bytes = 0;
    if (!mul_checked((uint64_t)N, (uint64_t)(K / B_OF(format)) * (uint64_t)S_OF(format), &bytes))
        return NQ_ERR_OVERFLOW;
    if (nbytes != bytes) return NQ_ERR_LENGTH_MISMATCH;
    return NQ_OK;
}

NQ_API int nq_gemv_q8_1(int32_t format, const void *weight, uint64_t nbytes, int64_t N, int64_t K,
                        const void *xq, int64_t M, float *y, hipStream_t stream) {
    const int st = nq_validate_gemv_q8_1(format, nbytes, N, K, M);
    if (st != NQ_OK) return st;
    if (!weight || !xq || !y) return NQ_ERR_NULL_ARG;
    if ((uintptr_t)xq % 4 != 0 || (uintptr_t)y % 4 != 0) return NQ_ERR_MISALIGNED;
    nq::GvLaunch L;
    L.w = (const uint8_t *)weight;
    L.N = (uint64_t)N;
    L.K = (uint64_t)K;
    L.M = (uint64_t)M;
    L.xq = (const uint8_t *)xq;
    L.y = y;
    L.cus = compute_units();
    return launch_gemv_family(format, L, stream);
}

NQ_API int nq_validate_gemm_q8_1(int32_t format, uint64_t nbytes, int64_t N, int64_t K, int64_t M) {
    if (format < 0 || format >= nq::NUM_FORMATS || TRAILER_OF(format) != 0) return NQ_ERR_UNKNOWN_FORMAT;
    if (N <= 0 || K <= 0 || M <= 0) return NQ_ERR_BAD_DIM;
    if (K % B_OF(format) != 0) return NQ_ERR_NOT_BLOCK_ALIGNED;
    if (N >= (1ll << 31) || K >= (1ll << 31) || M >= (1ll << 31)) return NQ_ERR_OVERFLOW;
    uint64_t bytes = 0, xbytes = 0, ybytes = 0;
    if (!mul_checked((uint64_t)M, (uint64_t)(K / 32) * 36u, &xbytes) || !mul_checked((uint64_t)M, (uint64_t)N * 4u, &ybytes))
        return NQ_ERR_OVERFLOW;
    if (!mul_checked((uint64_t)N, (uint64_t)(K / B_OF(format)) * (uint64_t)S_OF(format), &bytes))
        return NQ_ERR_OVERFLOW;
    if (nbytes != bytes) return NQ_ERR_LENGTH_MISMATCH;
    return NQ_OK;
}

NQ_API int nq_gemm_q8_1_workspace(int32_t format, int64_t N, int64_t K, int64_t M, uint64_t *bytes) {
    if (!bytes) return NQ_ERR_NULL_ARG;
    *bytes = 0;
    if (format < 0 || format >= nq::NUM_FORMATS || TRAILER_OF(format) != 0) return NQ_ERR_UNKNOWN_FORMAT;
    if (N <= 0 || K <= 0 || M <= 0) return NQ_ERR_BAD_DIM;
    if (K % B_OF(format) != 0) return NQ_ERR_NOT_BLOCK_ALIGNED;
    uint64_t wbytes = 0;
    if (N >= (1ll << 31) || K >= (1ll << 31) || M >= (1ll << 31) ||
        !mul_checked((uint64_t)N, (uint64_t)(K / B_OF(format)) * (uint64_t)S_OF(format), &wbytes))
        return NQ_ERR_OVERFLOW;
    const int st = nq_validate_gemm_q8_1(format, wbytes, N, K, M);
    if (st != NQ_OK) return st;
    if ((uint64_t)M >= nq::GM_MIN_M)
        *bytes = nq::gm_ws_layout(format, nq::gm_plan(format, (uint64_t)N, (uint64_t)K, (uint64_t)M, compute_units()),
                                  (uint64_t)N, (uint64_t)K, (uint64_t)M)
                     .total;
    return NQ_OK;
}

NQ_API int nq_gemm_q8_1(int32_t format, const void *weight, uint64_t nbytes, int64_t N, int64_t K,
                        const void *xq, int64_t M, float *y, void *workspace, uint64_t workspace_bytes,
                        hipStream_t stream) {
    const int st = nq_validate_gemm_q8_1(format, nbytes, N, K, M);
    if (st != NQ_OK) return st;
    if (!weight || !xq || !y) return NQ_ERR_NULL_ARG;
    if ((uintptr_t)xq % 4 != 0 || (uintptr_t)y % 4 != 0 || (uintptr_t)workspace % 16 != 0)
        return NQ_ERR_MISALIGNED;
    nq::GvLaunch L;
    L.w = (const uint8_t *)weight;
    L.N = (uint64_t)N;
    L.K = (uint64_t)K;
    L.M = (uint64_t)M;
    L.xq = (const uint8_t *)xq;
    L.y = y;
    L.cus = compute_units();
    if ((uint64_t)M >= nq::GM_MIN_M) {
        switch (REGISTRY[format].family) {
        case NQ_FAMILY_SIMPLE: return nq::launch_gemm_simple(format, L, workspace, workspace_bytes, stream);
        case NQ_FAMILY_KQUANT: return nq::launch_gemm_kquant(format, L, workspace, workspace_bytes, stream);
        case NQ_FAMILY_IQ: return nq::launch_gemm_iq(format, L, workspace, workspace_bytes, stream);
        default: return nq::launch_gemm_fp4t(format, L, workspace, workspace_bytes, stream);
        }
    }
    // fewer rows: the single-row kernel (one launch)
    for (int64_t m0 = 0; m0 < M; m0 += nq::GV_MAX_M) {
        nq::GvLaunch l = L;
        l.M = (uint64_t)(M - m0 < nq::GV_MAX_M ? M - m0 : nq::GV_MAX_M);
        l.xq = L.xq + (uint64_t)m0 * (uint64_t)(K / 32) * 36u;
        l.y = L.y + (uint64_t)m0 * (uint64_t)N;
        const int r = launch_gemv_family(format, l, stream);
        if (r != NQ_OK) return r;
    }
    return NQ_OK;
}

NQ_API const char *nq_status_string(int status) {
    switch (status) {
    case NQ_OK: return "ok";
    case NQ_ERR_NULL_ARG: return "a required pointer is NULL";
    case NQ_ERR_UNKNOWN_FORMAT: return "unknown format identifier";
    case NQ_ERR_BAD_RANK: return "shape rank must be at least 1";
    case NQ_ERR_BAD_DIM: return "a dimension or count is outside its allowed range";
    case NQ_ERR_NOT_BLOCK_ALIGNED: return "last dimension is not a multiple of the block size";
    case NQ_ERR_LENGTH_MISMATCH: return "payload length differs from the length rule";
    case NQ_ERR_OVERFLOW: return "byte or element count overflows";
    case NQ_ERR_BAD_DTYPE: return "unknown output dtype";
    case NQ_ERR_HIP: return "HIP launch failed";
    case NQ_ERR_BAD_DIVISORS: return "divisors must be in [1, 2^30] and divide the row count";
    case NQ_ERR_MISALIGNED: return "a pointer is not aligned as the call requires";
    case NQ_ERR_SCRATCH: return "the shape needs more workspace than the static scratch holds; use nq_gemm_q8_1";
    default: return "unknown status";
    }
}
