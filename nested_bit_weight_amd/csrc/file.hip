// file.hip -- on-disk form of a sliceable parent, host code only.
//
// One parent checkpoint serves every precision: the r-bit child keeps the
// most significant r bits of each code (MatGPTQ: Accurate and Efficient
// Post-Training Matryoshka Quantization, abstract) and loads exactly r bits
// per weight (MatGPTQ: Efficient and Accurate Inference over Nested Quantized
// Models, Abstract; Table 1, row "Exact r-bit loading").  The file puts the
// scales ahead of the planes and the planes MSB first, so the bytes an r-bit
// child needs are exactly a prefix of the parent's file: a loader reads
// nbw_file_prefix_bytes(n, k, r) bytes and nothing else, and a file cut
// after that many bytes is itself a valid r-bit child file.
//
// Layout (all integers little-endian):
//   [0, 4096)                  header (below), zero-padded
//   [4096, 4096 + S)           scales, bf16 [n][k/128] row-major, S = n*(k/128)*2
//   planes_offset              = 4096 + S rounded up to a multiple of 4096
//   planes_offset + p*PB       plane p (p = 0..7, 0 = MSB), PB = nbw_plane_bytes(n, k),
//                              byte for byte the device layout NBW_LAYOUT_T16
// Header fields (byte offset: type name):
//   0: char[8] magic "NBWPLAN1"; 8: u32 header bytes (4096); 12: u32 layout;
//   16: i64 n; 24: i64 k; 32: i32 planes written (8); 36: i32 group (128);
//   40: i64 plane bytes; 48: i64 scales offset; 56: i64 scales bytes;
//   64: i64 planes offset; 72: u32 scale type (1 = bf16); 76..4095: zero.
#include <cstring>

#include "nbw.h"

namespace {

constexpr char MAGIC[8] = {'N', 'B', 'W', 'P', 'L', 'A', 'N', '1'};
constexpr int64_t ALIGN = 4096;

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

template <typename T> void put(unsigned char *h, int off, T v) { std::memcpy(h + off, &v, sizeof v); }
template <typename T> T get(const unsigned char *h, int off) {
    T v;
    std::memcpy(&v, h + off, sizeof v);
    return v;
}

int64_t scales_bytes(int64_t n, int64_t k) { return n * (k / 128) * 2; }

}  // namespace

extern "C" {

int64_t nbw_file_prefix_bytes(int64_t n, int64_t k, int32_t r) {
    const int64_t pb = nbw_plane_bytes(n, k);
    if (pb < 0 || r < 0 || r > 8) return -1;
    return NBW_FILE_HEADER_BYTES + round_up(scales_bytes(n, k), ALIGN) + (int64_t)r * pb;
}

nbw_status nbw_file_header(int64_t n, int64_t k, void *header_out) {
    if (!header_out) return NBW_EINVAL;
    const int64_t pb = nbw_plane_bytes(n, k);
    if (pb < 0) return NBW_EINVAL;
    unsigned char *h = static_cast<unsigned char *>(header_out);
    std::memset(h, 0, NBW_FILE_HEADER_BYTES);
    std::memcpy(h, MAGIC, sizeof MAGIC);
    put<uint32_t>(h, 8, (uint32_t)NBW_FILE_HEADER_BYTES);
    put<uint32_t>(h, 12, (uint32_t)NBW_LAYOUT_T16);
    put<int64_t>(h, 16, n);
    put<int64_t>(h, 24, k);
    put<int32_t>(h, 32, 8);
    put<int32_t>(h, 36, 128);
    put<int64_t>(h, 40, pb);
    put<int64_t>(h, 48, NBW_FILE_HEADER_BYTES);
    put<int64_t>(h, 56, scales_bytes(n, k));
    put<int64_t>(h, 64, nbw_file_prefix_bytes(n, k, 0));
    put<uint32_t>(h, 72, 1u);
    return NBW_OK;
}

nbw_status nbw_file_parse(const void *header, int64_t file_bytes, nbw_file_info *info) {
    if (!header || !info) return NBW_EINVAL;
    const unsigned char *h = static_cast<const unsigned char *>(header);
    if (std::memcmp(h, MAGIC, sizeof MAGIC) != 0) return NBW_EINVAL;
    if (get<uint32_t>(h, 8) != (uint32_t)NBW_FILE_HEADER_BYTES) return NBW_EINVAL;
    if (get<uint32_t>(h, 12) != (uint32_t)NBW_LAYOUT_T16) return NBW_EUNSUPPORTED;
    if (get<uint32_t>(h, 72) != 1u || get<int32_t>(h, 36) != 128) return NBW_EUNSUPPORTED;
    const int64_t n = get<int64_t>(h, 16), k = get<int64_t>(h, 24);
    const int32_t nplanes = get<int32_t>(h, 32);
    const int64_t pb = nbw_plane_bytes(n, k);
    if (pb < 0 || nplanes < 1 || nplanes > 8) return NBW_EINVAL;
    // every derived field must be the one this layout fixes
    if (get<int64_t>(h, 40) != pb || get<int64_t>(h, 48) != NBW_FILE_HEADER_BYTES ||
        get<int64_t>(h, 56) != scales_bytes(n, k) ||
        get<int64_t>(h, 64) != nbw_file_prefix_bytes(n, k, 0))
        return NBW_EINVAL;
    const int64_t planes_offset = nbw_file_prefix_bytes(n, k, 0);
    if (file_bytes < planes_offset) return NBW_ERANGE;  // header and scales must be whole
    int64_t present = (file_bytes - planes_offset) / pb;
    if (present > nplanes) present = nplanes;
    info->n = n;
    info->k = k;
    info->nplanes = nplanes;
    info->layout = NBW_LAYOUT_T16;
    info->plane_bytes = pb;
    info->scales_offset = NBW_FILE_HEADER_BYTES;
    info->scales_bytes = scales_bytes(n, k);
    info->planes_offset = planes_offset;
    info->planes_present = (int32_t)present;
    info->reserved = 0;
    return NBW_OK;
}

}  // extern "C"
