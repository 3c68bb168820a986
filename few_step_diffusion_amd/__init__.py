"""MI355X-native hot path of a three-step video refiner (see include/fsd.h)."""
from .binding import *  # noqa: F401,F403
