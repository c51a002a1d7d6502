from .muonh_oracle import *  # noqa
