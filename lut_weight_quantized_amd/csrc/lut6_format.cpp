// Host side of the LUT-6 format: packing, unpacking, sizes and status names.
//
// Page "Clef-Flash-ANE-LUT6", section "LUT-6 text weights": four 6-bit
// indices are packed into three bytes, little-endian.  Reading: the three
// bytes are the 24-bit word w = i0 | i1<<6 | i2<<12 | i3<<18 (i0 = the lowest
// input column), stored low byte first.  Section "Weight precision": one
// 64-entry FP16 table per 16 output channels.
#include "lut6.h"

#include <stdint.h>

extern "C" size_t lut6_packed_bytes(int64_t N, int64_t K)
{
    if (N <= 0 || K <= 0 || K % 4) return 0;
    return (size_t)N * (size_t)(K / 4 * 3);
}

extern "C" size_t lut6_table_bytes(int64_t N)
{
    if (N <= 0 || N % 16) return 0;
    return (size_t)(N / 16) * 64 * 2;
}

extern "C" int lut6_pack(const uint8_t* idx, uint8_t* packed, int64_t N, int64_t K)
{
    if (!idx || !packed) return LUT6_E_NULL;
    if (N <= 0 || K <= 0 || K % 4) return LUT6_E_SHAPE;
    const int64_t groups = N * (K / 4);
    // refuse before writing anything
    for (int64_t i = 0; i < N * K; ++i)
        if (idx[i] > 63) return LUT6_E_INDEX_RANGE;
    for (int64_t gi = 0; gi < groups; ++gi) {
        const uint8_t* s = idx + 4 * gi;
        const uint32_t w = (uint32_t)s[0] | ((uint32_t)s[1] << 6) |
                           ((uint32_t)s[2] << 12) | ((uint32_t)s[3] << 18);
        uint8_t* d = packed + 3 * gi;
        d[0] = (uint8_t)w;
        d[1] = (uint8_t)(w >> 8);
        d[2] = (uint8_t)(w >> 16);
    }
    return LUT6_OK;
}

extern "C" int lut6_unpack(const uint8_t* packed, uint8_t* idx, int64_t N, int64_t K)
{
    if (!idx || !packed) return LUT6_E_NULL;
    if (N <= 0 || K <= 0 || K % 4) return LUT6_E_SHAPE;
    const int64_t groups = N * (K / 4);
    for (int64_t gi = 0; gi < groups; ++gi) {
        const uint8_t* s = packed + 3 * gi;
        const uint32_t w = (uint32_t)s[0] | ((uint32_t)s[1] << 8) | ((uint32_t)s[2] << 16);
        uint8_t* d = idx + 4 * gi;
        d[0] = (uint8_t)(w & 63);
        d[1] = (uint8_t)((w >> 6) & 63);
        d[2] = (uint8_t)((w >> 12) & 63);
        d[3] = (uint8_t)(w >> 18);
    }
    return LUT6_OK;
}

extern "C" const char* lut6_status_string(int status)
{
    switch (status) {
    case LUT6_OK: return "LUT6_OK";
    case LUT6_E_NULL: return "LUT6_E_NULL";
    case LUT6_E_SHAPE: return "LUT6_E_SHAPE";
    case LUT6_E_ALIGN: return "LUT6_E_ALIGN";
    case LUT6_E_SCALE: return "LUT6_E_SCALE";
    case LUT6_E_EPILOGUE: return "LUT6_E_EPILOGUE";
    case LUT6_E_INDEX_RANGE: return "LUT6_E_INDEX_RANGE";
    case LUT6_E_DEVICE: return "LUT6_E_DEVICE";
    case LUT6_E_ALIAS: return "LUT6_E_ALIAS";
    case LUT6_E_SCRATCH: return "LUT6_E_SCRATCH";
    default: return "LUT6_E_UNKNOWN";
    }
}
