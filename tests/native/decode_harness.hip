// Host-side harness for the library's bit-plane network (decode.h): runs the
// same pack / decode / extraction functions the kernels inline, on the CPU, with
// the kernels' chunk indexing, so tests can compare them with the oracle
// without a GPU.  Usage: decode_harness <pack|unpack|operands|bytes> n k r in out
// (bytes: the single-phase operands of the large-batch GEMM, r = 5..8, divided
// by 2^(8-r))
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "decode.h"

using namespace nbw;

static float bf16f(uint32_t h) {
    uint32_t u = (h & 0xFFFFu) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

template <int R>
static void byte_operands(const std::vector<uint8_t> &planes, int n, int k, std::vector<float> &vals) {
    if constexpr (R >= 5) {
        const int G = k / 128;
        const int64_t pb = (int64_t)((n + 15) / 16) * 16 * (k / 8);
        const float unit = (float)(1 << (8 - R));
        for (int row = 0; row < n; ++row)
            for (int g = 0; g < G; ++g) {
                const int64_t chunk = ((int64_t)(row / 16) * G + g) * 16 + row % 16;
                for (int d = 0; d < 4; ++d) {
                    uint32_t P[8] = {0};
                    for (int p = 0; p < R; ++p)
                        std::memcpy(&P[p], &planes[p * pb + chunk * 16 + 4 * d], 4);
                    uint32_t D[16];
                    decode_word_bytes<R>(P, D);
                    for (int m = 0; m < 16; ++m) {
                        const int64_t col = (int64_t)g * 128 + 32 * d + 2 * m;
                        vals[(int64_t)row * k + col] = bf16f(D[m]) / unit;
                        vals[(int64_t)row * k + col + 1] = bf16f(D[m] >> 16) / unit;
                    }
                }
            }
    }
}

template <int R>
static void unpack_or_operands(const std::vector<uint8_t> &planes, int n, int k, bool operands,
                               std::vector<uint8_t> &codes, std::vector<float> &vals) {
    const int G = k / 128;
    const int64_t pb = (int64_t)((n + 15) / 16) * 16 * (k / 8);
    for (int row = 0; row < n; ++row)
        for (int g = 0; g < G; ++g) {
            const int64_t chunk = ((int64_t)(row / 16) * G + g) * 16 + row % 16;
            for (int d = 0; d < 4; ++d) {
                uint32_t P[8] = {0};
                for (int p = 0; p < R; ++p)
                    std::memcpy(&P[p], &planes[p * pb + chunk * 16 + 4 * d], 4);
                constexpr int rp0 = Phases<R>::rp0, rp1 = Phases<R>::rp1;
                for (int m = 0; m < 16; ++m) {
                    const int64_t col = (int64_t)g * 128 + 32 * d + 2 * m;
                    if (!operands) {
                        uint32_t Z0[4], Z1[4];
                        network<rp0>(P, Z0);
                        uint32_t v = extract_codes<rp0>(Z0, m);
                        if constexpr (rp1 > 0) {
                            network<rp1>(P + 4, Z1);
                            v = (v << rp1) | extract_codes<rp1>(Z1, m);
                        }
                        codes[(int64_t)row * k + col] = (uint8_t)(v & 0xFF);
                        codes[(int64_t)row * k + col + 1] = (uint8_t)(v >> 16);
                    } else {
                        uint32_t D0[16], D1[16];
                        decode_word<R>(P, D0, D1);
                        uint32_t off0 = pick_offset_pair<rp0, Phases<R>::c0>(m);
                        float lo = bf16f(D0[m]) - bf16f(off0);
                        float hi = bf16f(D0[m] >> 16) - bf16f(off0 >> 16);
                        if constexpr (rp1 > 0) {
                            uint32_t off1 = pick_offset_pair<rp1, 0>(m);
                            lo += bf16f(D1[m]) - bf16f(off1);
                            hi += bf16f(D1[m] >> 16) - bf16f(off1 >> 16);
                        }
                        vals[(int64_t)row * k + col] = lo;
                        vals[(int64_t)row * k + col + 1] = hi;
                    }
                }
            }
        }
}

int main(int argc, char **argv) {
    if (argc != 7) return 2;
    const char *mode = argv[1];
    const int n = atoi(argv[2]), k = atoi(argv[3]), r = atoi(argv[4]);
    FILE *fi = fopen(argv[5], "rb");
    if (!fi) return 3;
    std::vector<uint8_t> in;
    uint8_t buf[1 << 16];
    size_t got;
    while ((got = fread(buf, 1, sizeof buf, fi)) > 0) in.insert(in.end(), buf, buf + got);
    fclose(fi);
    const int G = k / 128;
    const int64_t pb = (int64_t)((n + 15) / 16) * 16 * (k / 8);
    FILE *fo = fopen(argv[6], "wb");
    if (!fo) return 4;
    if (!strcmp(mode, "pack")) {
        std::vector<uint8_t> planes(8 * pb, 0);
        for (int tile = 0; tile < (n + 15) / 16; ++tile)
            for (int g = 0; g < G; ++g)
                for (int i = 0; i < 16; ++i) {
                    const int row = tile * 16 + i;
                    const int64_t chunk = ((int64_t)tile * G + g) * 16 + i;
                    for (int d = 0; d < 4; ++d) {
                        uint32_t W[8] = {0}, P[8];
                        if (row < n) std::memcpy(W, &in[(int64_t)row * k + g * 128 + 32 * d], 32);
                        pack_word32(W, P);
                        for (int p = 0; p < 8; ++p)
                            std::memcpy(&planes[p * pb + chunk * 16 + 4 * d], &P[p], 4);
                    }
                }
        fwrite(planes.data(), 1, planes.size(), fo);
    } else if (!strcmp(mode, "bytes")) {
        std::vector<float> vals((size_t)n * k);
        switch (r) {
        case 5: byte_operands<5>(in, n, k, vals); break;
        case 6: byte_operands<6>(in, n, k, vals); break;
        case 7: byte_operands<7>(in, n, k, vals); break;
        case 8: byte_operands<8>(in, n, k, vals); break;
        default: return 5;
        }
        fwrite(vals.data(), 4, vals.size(), fo);
    } else {
        const bool operands = !strcmp(mode, "operands");
        std::vector<uint8_t> codes((size_t)n * k);
        std::vector<float> vals(operands ? (size_t)n * k : 0);
        switch (r) {
        case 1: unpack_or_operands<1>(in, n, k, operands, codes, vals); break;
        case 2: unpack_or_operands<2>(in, n, k, operands, codes, vals); break;
        case 3: unpack_or_operands<3>(in, n, k, operands, codes, vals); break;
        case 4: unpack_or_operands<4>(in, n, k, operands, codes, vals); break;
        case 5: unpack_or_operands<5>(in, n, k, operands, codes, vals); break;
        case 6: unpack_or_operands<6>(in, n, k, operands, codes, vals); break;
        case 7: unpack_or_operands<7>(in, n, k, operands, codes, vals); break;
        case 8: unpack_or_operands<8>(in, n, k, operands, codes, vals); break;
        default: return 5;
        }
        if (operands) fwrite(vals.data(), 4, vals.size(), fo);
        else fwrite(codes.data(), 1, codes.size(), fo);
    }
    fclose(fo);
    return 0;
}
