// Small host-side entry points of the C ABI.
#include "gs_internal.h"

extern "C" const char* gs_error_string(int code) {
    switch (code) {
        case GS_OK: return "ok";
        case GS_EINVAL: return "invalid argument";
        case GS_EALIGN: return "pointer not 16-byte aligned";
        case GS_EWORKSPACE: return "workspace too small";
        case GS_EHIP: return "HIP kernel launch failed";
        case GS_ECAPACITY: return "size exceeds kernel indexing limits";
        default: return "unknown error";
    }
}

extern "C" int gs_version(void) { return 1; }

extern "C" int gs_tile_grid(const gs_camera* cam, int32_t* tx, int32_t* ty) {
    if (!gs::camera_ok(cam) || !tx || !ty) return GS_EINVAL;
    *tx = gs::tiles_x(cam);
    *ty = gs::tiles_y(cam);
    return GS_OK;
}
